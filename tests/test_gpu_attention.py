"""GPU parity of isd_kv_write and isd_attention against the oracle.

Tolerance: the pass criterion is 2e-3 relative for attention outputs (bf16
inputs, fp32 accumulation), read normwise per (sequence, query head) slab:
max |O - O*| / max |O*| over its rows x D. fp32 inputs are held to 1e-5.
"""

import copy

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload
from oracle import attention as ref

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to64(t):
    return t.detach().float().cpu().double().numpy()


def fill_cache(case):
    kv = dvd.KVCache(case.num_pages, case.Hkv, case.D, case.dtype, torch.from_numpy(case.table), DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write(kv, case.k_rows.to(DEV).contiguous(), case.v_rows.to(DEV).contiguous(),
                     torch.zeros(case.C, dtype=torch.int32, device=DEV),
                     torch.from_numpy(case.lengths.astype(np.int32)).to(DEV), dev_err=err)
    return kv, err


def oracle_pages(case):
    kp = np.zeros((case.num_pages, 16, case.Hkv, case.D))
    vp = np.zeros_like(kp)
    ref.kv_write(kp, vp, case.table, np.zeros(case.C, int), to64(case.k_rows), to64(case.v_rows), case.lengths)
    return kp, vp


def slab_errors(got, want):
    """max |got - want| / max |want| per (sequence, head)."""
    C, R, H, D = want.shape
    g = got.transpose(0, 2, 1, 3).reshape(C, H, R * D)
    w = want.transpose(0, 2, 1, 3).reshape(C, H, R * D)
    return np.abs(g - w).max(-1) / np.abs(w).max(-1)


def run(case, slices=0, seqs=None):
    print(f"attention case C={case.C} rows={case.rows} Hq={case.Hq} Hkv={case.Hkv} D={case.D} "
          f"{case.dtype} slices={slices}", flush=True)
    kv, err = fill_cache(case)
    out = dvd.isd_attention(kv, case.q.to(DEV), torch.from_numpy(case.ctx).to(DEV),
                            max_len=int(case.lengths.max()), slices=slices, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    got = out.cpu().double().numpy()
    kp, vp = oracle_pages(case)
    q64 = to64(case.q)
    if seqs is None:
        want = ref.block_attention(q64, kp, vp, case.table, case.ctx)
        return got, want
    want = ref.block_attention(q64[seqs], kp, vp, case.table[seqs], case.ctx[seqs])
    return got[seqs], want


def test_kv_write_matches_documented_page_layout():
    case = workload.AttentionCase(3, C=3, rows=8, Hq=8, Hkv=2, D=128, ctx=[0, 21, 50], spare_pages=3)
    kv, err = fill_cache(case)
    torch.cuda.synchronize()
    assert err.item() == 0
    kp, vp = oracle_pages(case)  # [P, 16, Hkv, D] plain layout
    P, Hkv, D = case.num_pages, case.Hkv, case.D
    k_dev = to64(kv.k_pages).reshape(P, Hkv, D // 8, 16, 8)
    v_dev = to64(kv.v_pages).reshape(P, Hkv, 2, D, 8)
    used = sorted(set(case.table[case.table >= 0].ravel().tolist()))
    for b in range(case.C):
        for t in range(int(case.lengths[b])):
            p, s = case.table[b, t // 16], t % 16
            assert np.array_equal(k_dev[p, :, :, s, :].reshape(Hkv, D), kp[p, s])
            assert np.array_equal(v_dev[p, :, s // 8, :, s % 8], vp[p, s])
    unused = sorted(set(range(P)) - set(used))
    assert unused and not k_dev[unused].any()


def test_tiny_fp32_config():
    """C=1, 8 rows (N=4), 4 query heads, 1 KV head, D=64, 128 cached, fp32."""
    case = workload.AttentionCase(0, C=1, rows=8, Hq=4, Hkv=1, D=64, ctx=128, dtype=torch.float32)
    got, want = run(case)
    assert slab_errors(got, want).max() < 1e-5


@pytest.mark.parametrize("slices", [0, 1, 3, 7, 41])
def test_bf16_gqa_ragged_contexts(slices):
    """8B-class heads (32/8, D=128), several tiles, ragged tails; slices
    from one workgroup for everything to several per sequence (merges)."""
    case = workload.AttentionCase(11, C=5, rows=8, Hq=32, Hkv=8, D=128, ctx=[0, 1, 31, 100, 1000])
    got, want = run(case, slices=slices)
    e = slab_errors(got, want)
    print("max slab error", e.max())
    assert e.max() < 2e-3


@pytest.mark.parametrize("N", [2, 3, 6, 8])
def test_32b_class_heads_strides(N):
    """64/8 heads: the GQA pack is 8 * 2N query rows (16..128)."""
    case = workload.AttentionCase(20 + N, C=2, rows=2 * N, Hq=64, Hkv=8, D=128, ctx=[333, 1290])
    got, want = run(case, slices=5)
    assert slab_errors(got, want).max() < 2e-3


def test_head_dim_64_bf16_and_single_token_context():
    case = workload.AttentionCase(31, C=3, rows=8, Hq=8, Hkv=2, D=64, ctx=[0, 5, 77])
    got, want = run(case)
    assert slab_errors(got, want).max() < 2e-3
    # row 0 of a sequence without context sees exactly its own value row
    v0 = to64(case.v_rows[0, 0])
    for h in range(8):
        assert np.allclose(got[0, 0, h], v0[h // 4], rtol=1e-6, atol=1e-6)


def test_largest_query_pack_and_rows():
    """rows = 64 with group 2 (128 query columns)."""
    case = workload.AttentionCase(41, C=2, rows=64, Hq=4, Hkv=2, D=128, ctx=[10, 300])
    got, want = run(case, slices=9)
    assert slab_errors(got, want).max() < 2e-3


def test_stationary_batch_shapes_sampled():
    """C=64, N=4, 32/8 heads, D=128, contexts U{1024..8192}, 16-token pages in
    a shuffled pool: the whole batch runs, 6 sampled sequences are checked."""
    case = workload.AttentionCase(3, C=64, rows=8, Hq=32, Hkv=8, D=128, ctx=("uniform", 1024, 8192))
    seqs = np.array([0, 9, 17, 31, 48, 63])
    got, want = run(case, seqs=seqs)
    assert slab_errors(got, want).max() < 2e-3


def test_outputs_are_deterministic():
    case = workload.AttentionCase(5, C=4, rows=8, Hq=32, Hkv=8, D=128, ctx=[700, 2000, 64, 3000])
    kv, err = fill_cache(case)
    q, ctx = case.q.to(DEV), torch.from_numpy(case.ctx).to(DEV)
    a = dvd.isd_attention(kv, q, ctx, max_len=3008, slices=13)
    b = dvd.isd_attention(kv, q, ctx, max_len=3008, slices=13)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bad_page_id_sets_device_flag():
    case = workload.AttentionCase(6, C=2, rows=8, Hq=8, Hkv=2, D=128, ctx=[40, 40])
    kv, err = fill_cache(case)
    torch.cuda.synchronize()
    assert err.item() == 0
    kv.block_table[1, 1] = case.num_pages + 5
    dvd.isd_attention(kv, case.q.to(DEV), torch.from_numpy(case.ctx).to(DEV), max_len=48, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & dvd.DEV_PAGE_OOB


@pytest.mark.parametrize("slices", [0, dvd.attn_invariant(8), dvd.attn_invariant(4), dvd.attn_invariant(1)])
def test_8b_single_sequence_context_4096(slices):
    """C=1, N=4, 32/8 heads, D=128, 4096 cached tokens: every output checked,
    in the stream-K split and in the batch-invariant split with chunks of 8
    tiles (the single-sequence step's launch), 4 and 1 tile."""
    case = workload.AttentionCase(2, C=1, rows=8, Hq=32, Hkv=8, D=128, ctx=4096)
    got, want = run(case, slices=slices)
    assert slab_errors(got, want).max() < 2e-3


@pytest.mark.parametrize("t", [8, 4, 1])
def test_single_sequence_equals_its_rows_in_a_wide_batch(t):
    """A single sequence runs on a grid of its own shape (few chunks: one KV
    head per workgroup) and a 64-sequence batch on another (eight heads per
    workgroup); the sequence's rows come out bit for bit the same in both,
    with the batch-invariant split."""
    C, rows = 64, 8
    ctx = np.full(C, 1024, np.int64)
    ctx[17] = 4096
    case = workload.AttentionCase(12, C=C, rows=rows, Hq=32, Hkv=8, D=128, ctx=ctx)
    print(f"single sequence in a batch t={t}", flush=True)
    kv, err = fill_cache(case)
    max_len = int(case.lengths.max())
    ctx_d = torch.from_numpy(case.ctx.astype(np.int32)).to(DEV)
    q = case.q.to(DEV)
    inv = dvd.attn_invariant(t)
    batch = dvd.isd_attention(kv, q, ctx_d, max_len=max_len, slices=inv, dev_err=err)
    solo_kv = copy.copy(kv)
    solo_kv.block_table = kv.block_table[17:18].contiguous()
    solo = dvd.isd_attention(solo_kv, q[17:18].contiguous(), ctx_d[17:18].contiguous(), max_len=max_len,
                             slices=inv, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(solo), bits(batch[17:18]))
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q)[17:18], kp, vp, case.table[17:18], case.ctx[17:18])
    assert slab_errors(solo.cpu().double().numpy(), want).max() < 2e-3


@pytest.mark.parametrize("N", [2, 3, 4, 6, 8])
def test_32b_stride_sweep_shapes(N):
    """C=16, 64/8 heads, D=128, contexts of 16,384 tokens, block of 2N rows:
    the whole batch runs, two sequences are checked in full."""
    case = workload.AttentionCase(50 + N, C=16, rows=2 * N, Hq=64, Hkv=8, D=128, ctx=16384)
    got, want = run(case, seqs=np.array([3, 12]))
    assert slab_errors(got, want).max() < 2e-3


def bits(t):
    return t.contiguous().view(-1).view(torch.int32)


@pytest.mark.parametrize("t,Hq,dtype", [(1, 32, torch.bfloat16), (4, 32, torch.bfloat16),
                                         (4, 64, torch.bfloat16), (64, 32, torch.bfloat16),
                                         (4, 32, torch.float32)])
def test_invariant_split_rows_equal_one_row_calls(t, Hq, dtype):
    """Batch-invariant split: row i of every stride block equals, bit for bit,
    the same query sent as a one-row call with ctx + i cached tokens (the AR
    forward), whether those calls are batched together, reordered, or one
    sequence alone. Contexts put blocks across chunk boundaries (32t - 3),
    on them (32t), and make sequences of many chunks."""
    C, rows, D = 7, 8, 128
    ctx = [0, 5, 32 * t - 3, 32 * t, 3 * 32 * t - 1, 700, 2100]
    case = workload.AttentionCase(41 + t, C=C, rows=rows, Hq=Hq, Hkv=8, D=D, ctx=ctx, dtype=dtype)
    print(f"invariant split t={t} Hq={Hq} {dtype} ctx={ctx}", flush=True)
    kv, err = fill_cache(case)
    max_len = int(case.lengths.max())
    ctx_d = torch.from_numpy(case.ctx).to(DEV)
    q = case.q.to(DEV)
    inv = dvd.attn_invariant(t)
    blk = dvd.isd_attention(kv, q, ctx_d, max_len=max_len, slices=inv, dev_err=err)

    # every row as its own one-row sequence over its sequence's pages
    ar = copy.copy(kv)
    ar.block_table = kv.block_table.repeat_interleave(rows, dim=0).contiguous()
    ctx1 = (ctx_d[:, None] + torch.arange(rows, device=DEV, dtype=torch.int32)[None, :]).reshape(-1).contiguous()
    q1 = q.reshape(C * rows, 1, Hq, D).contiguous()
    one = dvd.isd_attention(ar, q1, ctx1, max_len=max_len, slices=inv, dev_err=err)
    # the same one-row calls in reverse order, with a larger max_len
    rev = torch.arange(C * rows - 1, -1, -1, device=DEV)
    ar_r = copy.copy(kv)
    ar_r.block_table = ar.block_table[rev].contiguous()
    one_r = dvd.isd_attention(ar_r, q1[rev].contiguous(), ctx1[rev].contiguous(), max_len=max_len + 500,
                              slices=inv, dev_err=err)
    # the longest sequence alone, as a block
    solo_kv = copy.copy(kv)
    solo_kv.block_table = kv.block_table[C - 1:].contiguous()
    solo = dvd.isd_attention(solo_kv, q[C - 1:].contiguous(), ctx_d[C - 1:].contiguous(), max_len=max_len,
                             slices=inv, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(blk), bits(one))
    assert torch.equal(bits(one_r), bits(one[rev]))
    assert torch.equal(bits(solo), bits(blk[C - 1:]))
    # and it is the attention the oracle computes
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q), kp, vp, case.table, case.ctx)
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    assert slab_errors(blk.cpu().double().numpy(), want).max() < tol


def test_invariant_split_flags_sequences_beyond_max_len():
    """Chunked split with max_len below a sequence's length: that sequence is
    left unwritten and ISD_DEV_CAPACITY is flagged; the others are exact."""
    case = workload.AttentionCase(47, C=3, rows=8, Hq=8, Hkv=2, D=64, ctx=[0, 100, 500])
    kv, err = fill_cache(case)
    out = torch.full((3, 8, 8, 64), 7.0, device=DEV)
    dvd.isd_attention(kv, case.q.to(DEV), torch.from_numpy(case.ctx).to(DEV), max_len=120,
                      slices=dvd.attn_invariant(2), out=out, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 2  # ISD_DEV_CAPACITY
    got = out.cpu().double().numpy()
    assert (got[2] == 7.0).all()
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q[:2]), kp, vp, case.table[:2], case.ctx[:2])
    assert slab_errors(got[:2], want).max() < 2e-3


def test_invariant_split_at_the_bench_shape_sampled_rows():
    """The stationary-batch shape (C=64, 8-row blocks, 32/8 heads, ragged
    1K-8K contexts) in the batch-invariant split with 64-tile chunks: every
    row of a sample of 16 sequences equals, bit for bit, its one-row call
    with ctx + i cached tokens made as a separate batch."""
    C, rows, t = 64, 8, 64
    case = workload.AttentionCase(3, C=C, rows=rows, Hq=32, Hkv=8, D=128, ctx=("uniform", 1024, 8192))
    print(f"invariant split at C={C}", flush=True)
    kv, err = fill_cache(case)
    max_len = int(case.lengths.max())
    ctx_d = torch.from_numpy(case.ctx).to(DEV)
    q = case.q.to(DEV)
    blk = dvd.isd_attention(kv, q, ctx_d, max_len=max_len, slices=dvd.attn_invariant(t), dev_err=err)
    seqs = torch.from_numpy(np.random.default_rng(9).choice(C, 16, replace=False)).to(DEV)
    ar = copy.copy(kv)
    ar.block_table = kv.block_table[seqs].repeat_interleave(rows, dim=0).contiguous()
    ctx1 = (ctx_d[seqs][:, None] + torch.arange(rows, device=DEV, dtype=torch.int32)[None, :]).reshape(-1).contiguous()
    q1 = q[seqs].reshape(16 * rows, 1, 32, 128).contiguous()
    one = dvd.isd_attention(ar, q1, ctx1, max_len=max_len, slices=dvd.attn_invariant(t), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(blk[seqs]), bits(one))


def block_rows(case, dev=DEV):
    """The block's own K/V rows [C, rows, Hkv, D] (positions ctx .. ctx+rows-1)."""
    k = torch.stack([case.k_rows[b, int(c):int(c) + case.rows] for b, c in enumerate(case.ctx)])
    v = torch.stack([case.v_rows[b, int(c):int(c) + case.rows] for b, c in enumerate(case.ctx)])
    return k.to(dev).contiguous(), v.to(dev).contiguous()


@pytest.mark.parametrize("slices,dtype", [(0, torch.bfloat16), (5, torch.bfloat16),
                                          (dvd.attn_invariant(1), torch.bfloat16),
                                          (dvd.attn_invariant(2), torch.bfloat16), (0, torch.float32)])
def test_attention_with_block_equals_write_then_attend(slices, dtype):
    """isd_attention_with_block over pages that hold only the cached context
    equals isd_kv_write of the block followed by isd_attention, bit for bit,
    and leaves the pages as they were. Contexts put blocks across page (16),
    tile (32) and chunk (32t) boundaries, with empty and one-token caches."""
    D = 128 if dtype == torch.bfloat16 else 64
    case = workload.AttentionCase(71, C=6, rows=8, Hq=32, Hkv=8, D=D, ctx=[0, 1, 28, 60, 125, 250], dtype=dtype)
    print(f"attention with block slices={slices} {dtype}", flush=True)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    zeros = torch.zeros(case.C, dtype=torch.int32, device=DEV)
    kb, vb = block_rows(case)
    max_len = int(case.lengths.max())
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv = dvd.KVCache(case.num_pages, case.Hkv, case.D, dtype, torch.from_numpy(case.table), DEV)
    dvd.isd_kv_write(kv, case.k_rows.to(DEV).contiguous(), case.v_rows.to(DEV).contiguous(), zeros, ctx, dev_err=err)
    torch.cuda.synchronize()
    before = kv.k_pages.clone(), kv.v_pages.clone()
    got = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=max_len, slices=slices, dev_err=err, k_blk=kb, v_blk=vb)
    torch.cuda.synchronize()
    assert torch.equal(kv.k_pages, before[0]) and torch.equal(kv.v_pages, before[1])
    dvd.isd_kv_write(kv, kb, vb, ctx, dev_err=err)
    want = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=max_len, slices=slices, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(got), bits(want))
    kp, vp = oracle_pages(case)
    ref_out = ref.block_attention(to64(case.q), kp, vp, case.table, case.ctx)
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    assert slab_errors(got.cpu().double().numpy(), ref_out).max() < tol


def test_attention_with_block_needs_pages_only_below_ctx():
    """Block-table entries past the cached context are -1 (no page yet): no
    error is flagged and the output is the oracle's."""
    case = workload.AttentionCase(73, C=3, rows=8, Hq=8, Hkv=2, D=64, ctx=[16, 40, 100])
    table = case.table.copy()
    for b, c in enumerate(case.ctx):
        table[b, -(-int(c) // 16):] = -1  # pages wholly past the context
    kv = dvd.KVCache(case.num_pages, case.Hkv, case.D, case.dtype, torch.from_numpy(table), DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    dvd.isd_kv_write(kv, case.k_rows.to(DEV).contiguous(), case.v_rows.to(DEV).contiguous(),
                     torch.zeros(case.C, dtype=torch.int32, device=DEV), ctx, dev_err=err)
    kb, vb = block_rows(case)
    for slices in (0, dvd.attn_invariant(1)):
        got = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=int(case.lengths.max()), slices=slices,
                                dev_err=err, k_blk=kb, v_blk=vb)
        torch.cuda.synchronize()
        assert err.item() == 0
        kp, vp = oracle_pages(case)
        want = ref.block_attention(to64(case.q), kp, vp, case.table, case.ctx)
        assert slab_errors(got.cpu().double().numpy(), want).max() < 2e-3


def test_attention_with_block_rows_equal_one_row_calls():
    """Lossless R-ISD with the block read from its rows: row i of a block
    call equals the one-row call at ctx + i (earlier rows already in the
    pages, its own row from the block), bit for bit, in the invariant split."""
    t, C, rows, Hq, D = 2, 5, 8, 32, 128
    case = workload.AttentionCase(74, C=C, rows=rows, Hq=Hq, Hkv=8, D=D, ctx=[0, 30, 61, 64, 200])
    kv, err = fill_cache(case)  # every position, so the one-row calls find rows < ctx + i in the pages
    ctx = torch.from_numpy(case.ctx).to(DEV)
    kb, vb = block_rows(case)
    inv = dvd.attn_invariant(t)
    max_len = int(case.lengths.max())
    blk = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=max_len, slices=inv, dev_err=err, k_blk=kb, v_blk=vb)
    ar = copy.copy(kv)
    ar.block_table = kv.block_table.repeat_interleave(rows, dim=0).contiguous()
    ctx1 = (ctx[:, None] + torch.arange(rows, device=DEV, dtype=torch.int32)[None, :]).reshape(-1).contiguous()
    q1 = case.q.to(DEV).reshape(C * rows, 1, Hq, D).contiguous()
    one = dvd.isd_attention(ar, q1, ctx1, max_len=max_len, slices=inv, dev_err=err,
                            k_blk=kb.reshape(C * rows, 1, 8, D).contiguous(), v_blk=vb.reshape(C * rows, 1, 8, D).contiguous())
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(blk), bits(one))


def test_kv_write_layers_equals_per_layer_calls():
    """Three layers in one stacked allocation, committed in one launch with
    per-sequence start and row counts, equal three isd_kv_write calls."""
    L, C, rows, Hkv, D = 3, 4, 8, 8, 128
    case = workload.AttentionCase(75, C=C, rows=rows, Hq=8, Hkv=Hkv, D=D, ctx=[3, 17, 40, 64], headroom=8)
    caches, stride = dvd.KVCache.stacked(L, case.num_pages, Hkv, D, torch.bfloat16, torch.from_numpy(case.table), DEV)
    k = workload.normal((L, C, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 75, "lk").to(DEV)
    v = workload.normal((L, C, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 75, "lv").to(DEV)
    pos0 = torch.from_numpy(case.ctx).to(DEV)
    nrows = torch.tensor([8, 3, 1, 0], dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write_layers(caches[0], stride, k, v, pos0, nrows, dev_err=err)
    for l in range(L):
        ref_kv = dvd.KVCache(case.num_pages, Hkv, D, torch.bfloat16, torch.from_numpy(case.table), DEV)
        dvd.isd_kv_write(ref_kv, k[l].contiguous(), v[l].contiguous(), pos0, nrows, dev_err=err)
        torch.cuda.synchronize()
        assert torch.equal(caches[l].k_pages.view(torch.int16), ref_kv.k_pages.view(torch.int16))
        assert torch.equal(caches[l].v_pages.view(torch.int16), ref_kv.v_pages.view(torch.int16))
    assert err.item() == 0


@pytest.mark.parametrize("shape", ["8b", "8b1", "32b"])
def test_timed_launch_configuration_against_the_oracle(shape):
    """The call the step benchmark times, at its full shapes: the block's K/V
    read from its rows (pages hold only the cached context), the
    batch-invariant split with 64-tile chunks (8B: C=64, 32/8 heads, ragged
    1K-8K contexts), 8-tile chunks (8B, one sequence of 4,096 cached tokens)
    or 66-tile chunks (32B: C=16, 64/8 heads, 16,384 cached tokens). The
    whole batch runs and every sequence is checked against the oracle in
    full."""
    if shape == "8b":
        case = workload.AttentionCase(81, C=64, rows=8, Hq=32, Hkv=8, D=128, ctx=("uniform", 1024, 8192))
        t = 64
    elif shape == "8b1":
        case = workload.AttentionCase(83, C=1, rows=8, Hq=32, Hkv=8, D=128, ctx=4096)
        t = 8
    else:
        case = workload.AttentionCase(82, C=16, rows=8, Hq=64, Hkv=8, D=128, ctx=16384)
        t = 66
    seqs = np.arange(case.C)
    print(f"timed launch configuration {shape} t={t}", flush=True)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv = dvd.KVCache(case.num_pages, case.Hkv, case.D, case.dtype, torch.from_numpy(case.table), DEV)
    dvd.isd_kv_write(kv, case.k_rows.to(DEV).contiguous(), case.v_rows.to(DEV).contiguous(),
                     torch.zeros(case.C, dtype=torch.int32, device=DEV), ctx, dev_err=err)
    kb, vb = block_rows(case)
    got = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=int(case.lengths.max()), slices=dvd.attn_invariant(t),
                            dev_err=err, k_blk=kb, v_blk=vb)
    torch.cuda.synchronize()
    assert err.item() == 0
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q)[seqs], kp, vp, case.table[seqs], case.ctx[seqs])
    assert slab_errors(got.cpu().double().numpy()[seqs], want).max() < 2e-3


@pytest.mark.parametrize("split", ["chunked", "stream-K"])
def test_bad_sequences_inside_the_batch_leave_the_others_exact(split):
    """A sequence with ctx = -1 (ISD_DEV_STATE) sits in the middle of the
    batch and, in the chunked split, another one exceeds max_len
    (ISD_DEV_CAPACITY): both have no work, so the chunks or tiles of every
    later sequence move to other workgroups. The flags are raised and every
    other sequence matches the oracle."""
    case = workload.AttentionCase(48, C=5, rows=8, Hq=8, Hkv=2, D=64, ctx=[300, 50, 2000, 900, 64])
    kv, err = fill_cache(case)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    ctx[1] = -1
    chunked = split == "chunked"
    out = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=1000 if chunked else int(case.lengths.max()),
                            slices=dvd.attn_invariant(2) if chunked else 0, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == (dvd.DEV_STATE | dvd.DEV_CAPACITY if chunked else dvd.DEV_STATE)
    good = np.array([0, 3, 4] if chunked else [0, 2, 3, 4])
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q)[good], kp, vp, case.table[good], case.ctx[good])
    assert slab_errors(out.cpu().double().numpy()[good], want).max() < 2e-3


@pytest.mark.parametrize("slices,with_block", [(0, False), (5, False), (dvd.attn_invariant(1), False),
                                               (dvd.attn_invariant(2), True), (0, True)])
def test_bf16_output_is_the_rounded_fp32_output(slices, with_block):
    """odtype bf16 stores the fp32 result rounded to nearest even, bit for
    bit, whether a (sequence, head) is finished in the main kernel (one
    piece) or by the merge of several pieces: contexts from 0 to 700 tokens
    give both kinds in one call."""
    case = workload.AttentionCase(73, C=7, rows=8, Hq=32, Hkv=8, D=128, ctx=[0, 1, 31, 64, 129, 300, 700],
                                  dtype=torch.bfloat16)
    print(f"attention bf16 output slices={slices} with_block={with_block}", flush=True)
    kv, err = fill_cache(case)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    q = case.q.to(DEV)
    extra = {}
    if with_block:
        extra = dict(zip(("k_blk", "v_blk"), block_rows(case)))
    max_len = int(case.lengths.max())
    f32 = dvd.isd_attention(kv, q, ctx, max_len=max_len, slices=slices, dev_err=err, **extra)
    b16 = dvd.isd_attention(kv, q, ctx, max_len=max_len, slices=slices, dev_err=err, odtype=torch.bfloat16, **extra)
    torch.cuda.synchronize()
    assert err.item() == 0 and b16.dtype == torch.bfloat16
    assert torch.equal(b16.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16))
    kp, vp = oracle_pages(case)
    want = ref.block_attention(to64(case.q), kp, vp, case.table, case.ctx)
    assert slab_errors(b16.cpu().double().numpy(), want).max() < 2e-3 + 2.0 ** -8

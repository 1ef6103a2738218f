"""Pins of the oracle's paged KV write and block attention (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import attention

import workload


def build_pages(case):
    """Oracle-side pages from a seeded case, written with the oracle's own
    KV write (plain [P, 16, Hkv, D] layout)."""
    C, Hkv, D = case.C, case.Hkv, case.D
    kp = np.full((case.num_pages, workload.PAGE_SIZE, Hkv, D), np.nan)
    vp = np.full_like(kp, np.nan)
    attention.kv_write(kp, vp, case.table, np.zeros(C, int),
                       case.k_rows.double().numpy(), case.v_rows.double().numpy(),
                       case.lengths)
    return kp, vp


def brute(q, K, V, ctx, scale):
    """Pure-Python loops for one sequence: K, V logical [L, Hkv, D]."""
    R, Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.zeros((R, Hq, D))
    for i in range(R):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = [sum(q[i, h, d] * K[t, g, d] for d in range(D)) * scale
                 for t in range(ctx + i + 1)]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            z = sum(e)
            for d in range(D):
                out[i, h, d] = sum(e[t] * V[t, g, d] for t in range(len(e))) / z
    return out


def test_kv_write_then_gather_round_trips():
    case = workload.AttentionCase(1, C=3, rows=8, Hq=4, Hkv=2, D=8, ctx=[0, 17, 40],
                                  dtype=torch.float32, spare_pages=5)
    kp, vp = build_pages(case)
    for b in range(case.C):
        L = int(case.lengths[b])
        got = attention.gather_sequence(kp, case.table[b], L)
        assert np.array_equal(got, case.k_rows[b, :L].double().numpy())
    # untouched pages stay unwritten
    used = set(case.table[case.table >= 0].ravel().tolist())
    for p in set(range(case.num_pages)) - used:
        assert np.isnan(kp[p]).all()


def test_block_attention_matches_brute_force():
    case = workload.AttentionCase(2, C=2, rows=4, Hq=4, Hkv=2, D=6, ctx=[5, 13],
                                  dtype=torch.float32)
    kp, vp = build_pages(case)
    scale = 0.37
    got = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx, scale)
    for b in range(case.C):
        L = int(case.lengths[b])
        K = case.k_rows[b, :L].double().numpy()
        V = case.v_rows[b, :L].double().numpy()
        want = brute(case.q[b].double().numpy(), K, V, int(case.ctx[b]), scale)
        assert np.allclose(got[b], want, rtol=1e-12, atol=1e-12)


def test_block_attention_matches_torch_sdpa_fp64():
    """Tiny fp32 config: C=1, 8 rows, 4 query heads, 1 KV head, D=64,
    128 cached tokens; the library routine takes an explicit mask."""
    case = workload.AttentionCase(0, C=1, rows=8, Hq=4, Hkv=1, D=64, ctx=128,
                                  dtype=torch.float32)
    kp, vp = build_pages(case)
    got = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    L = int(case.lengths[0])
    q = case.q[0].double().permute(1, 0, 2)                      # [Hq, R, D]
    k = case.k_rows[0, :L].double().permute(1, 0, 2).expand(4, L, 64)
    v = case.v_rows[0, :L].double().permute(1, 0, 2).expand(4, L, 64)
    mask = torch.arange(L)[None, :] <= (128 + torch.arange(8))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    assert np.allclose(got[0], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_first_row_without_context_returns_first_value():
    case = workload.AttentionCase(4, C=1, rows=8, Hq=2, Hkv=1, D=16, ctx=0, dtype=torch.float32)
    kp, vp = build_pages(case)
    got = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    v0 = case.v_rows[0, 0, 0].double().numpy()
    assert np.array_equal(got[0, 0, 0], v0) and np.array_equal(got[0, 0, 1], v0)


def test_equal_keys_give_mean_of_visible_values():
    case = workload.AttentionCase(5, C=1, rows=4, Hq=2, Hkv=1, D=8, ctx=9, dtype=torch.float32)
    case.k_rows[:] = case.k_rows[:, :1]
    kp, vp = build_pages(case)
    got = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    for i in range(4):
        mean = case.v_rows[0, :10 + i, 0].double().mean(0).numpy()
        assert np.allclose(got[0, i, 1], mean, rtol=1e-12, atol=1e-13)


def test_gqa_is_mha_with_repeated_kv_heads():
    case = workload.AttentionCase(6, C=2, rows=6, Hq=4, Hkv=2, D=8, ctx=[3, 20], dtype=torch.float32)
    kp, vp = build_pages(case)
    got = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    kp2 = np.repeat(kp, 2, axis=2)
    vp2 = np.repeat(vp, 2, axis=2)
    mha = attention.block_attention(case.q.double().numpy(), kp2, vp2, case.table, case.ctx)
    assert np.array_equal(got, mha)


def test_block_rows_see_earlier_block_rows_only():
    """Changing the K/V of block row 5 must leave rows 0..4 untouched."""
    case = workload.AttentionCase(7, C=1, rows=8, Hq=2, Hkv=1, D=8, ctx=30, dtype=torch.float32)
    kp, vp = build_pages(case)
    a = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    case.k_rows[0, 35] += 3.0
    case.v_rows[0, 35] -= 2.0
    kp, vp = build_pages(case)
    b = attention.block_attention(case.q.double().numpy(), kp, vp, case.table, case.ctx)
    assert np.array_equal(a[0, :5], b[0, :5]) and not np.allclose(a[0, 5:], b[0, 5:])

"""Pins of the oracle's forward pieces (CPU only): RMSNorm, SiLU / SwiGLU,
bf16 rounding and the decoder block composed from the pinned modules."""

import math

import numpy as np
import torch

import workload
from oracle import attention, forward, lora


def test_rmsnorm_brute_force_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 37)) * 3
    g = rng.normal(size=37)
    y = forward.rmsnorm(x, g)
    for i in range(5):
        r = math.sqrt(sum(v * v for v in x[i]) / 37 + forward.EPS)
        for j in range(37):
            assert abs(y[i, j] - x[i, j] / r * g[j]) < 1e-12
    # with unit gain the output's mean square is 1 (up to eps)
    u = forward.rmsnorm(x, np.ones(37))
    assert np.allclose(np.mean(u * u, axis=1), 1.0, atol=1e-6)
    # scaling a row does not change its normalised value (eps aside)
    assert np.allclose(forward.rmsnorm(7.5 * x, g), y, atol=1e-6)


def test_silu_and_swiglu_closed_forms():
    z = np.array([-40.0, -1.0, 0.0, 0.5, 2.0, 40.0])
    s = forward.silu(z)
    for zi, si in zip(z, s):
        assert abs(si - zi / (1 + math.exp(-zi))) < 1e-15
    assert s[2] == 0.0 and abs(s[-1] - 40.0) < 1e-12 and abs(s[0]) < 1e-15
    up = np.array([1.0, 2.0, 3.0, -1.0, 0.25, 0.0])
    assert np.allclose(forward.swiglu(z, up), s * up)


def test_bf16_rounding_ties_to_even():
    e = 2.0 ** -8  # half a bf16 ulp at 1.0 is 2^-8
    vals = np.array([1.0, 1.0 + e, 1.0 + 3 * e, 1.0 + 2 * e, -1.0 - e, 3.0e38])
    want = np.array([1.0, 1.0, 1.0 + 4 * e, 1.0 + 2 * e, -1.0, 3.0e38])
    got = forward.bf16_round(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: the even mantissa (1) wins;
    # 1 + 3 * 2^-8 rounds up; 1 + 2^-7 is representable
    assert np.array_equal(got[:5], want[:5])
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8


def small_model(seed, H=64, Hq=4, Hkv=2, D=16, I=96, r=16):
    rng = np.random.default_rng(seed)
    nq = (Hq + 2 * Hkv) * D
    p = dict(Hq=Hq, Hkv=Hkv, D=D,
             g1=rng.normal(1, 0.1, H), g2=rng.normal(1, 0.1, H),
             Wqkv=rng.normal(0, 0.1, (nq, H)), Aqkv=rng.normal(0, 0.05, (r, H)), Bqkv=rng.normal(0, 0.05, (nq, r)),
             Wo=rng.normal(0, 0.1, (H, Hq * D)), Ao=rng.normal(0, 0.05, (r, Hq * D)), Bo=rng.normal(0, 0.05, (H, r)),
             Wgu=rng.normal(0, 0.1, (2 * I, H)), Wd=rng.normal(0, 0.1, (H, I)))
    return p


def test_block_is_the_composition_of_its_pinned_parts():
    """With the MLP switched off (Wd = 0) the block adds exactly the O
    projection of the attention of its own q/k/v; with Wo = 0 as well it
    returns h unchanged; clean rows do not see the adapter."""
    C, N, H = 2, 2, 64
    R, M = 2 * N, 2 * 2 * N
    p = small_model(1, H=H)
    rng = np.random.default_rng(2)
    h = rng.normal(size=(M, H))
    ctx = np.array([3, 17])
    table, num_pages = workload.block_table(5, ctx + R)
    kp = np.zeros((num_pages, 16, p["Hkv"], p["D"]))
    vp = np.zeros_like(kp)
    cached_k = rng.normal(size=(C, int(ctx.max()), p["Hkv"], p["D"]))
    cached_v = rng.normal(size=cached_k.shape)
    attention.kv_write(kp, vp, table, np.zeros(C, int), cached_k, cached_v, ctx)
    mask = workload.stride_mask(M, N)
    p0 = dict(p, Wd=np.zeros_like(p["Wd"]))
    out, mid = forward.block(h, p0, (kp, vp, table), ctx, mask, N)
    assert np.array_equal(mid["d"], np.zeros_like(mid["d"]))
    o_proj = lora.gated_lora(mid["ob"], p["Wo"], p["Ao"], p["Bo"], mask, 1.0)
    assert np.array_equal(out, h + o_proj)
    # attention of the block's own q/k/v over cache + block
    kp2, vp2 = kp.copy(), vp.copy()
    attention.kv_write(kp2, vp2, table, ctx, mid["k"], mid["v"], np.full(C, R))
    assert np.allclose(mid["o"], attention.block_attention(mid["q"], kp2, vp2, table, ctx))
    out2, _ = forward.block(h, dict(p0, Wo=np.zeros_like(p["Wo"]), Bo=np.zeros_like(p["Bo"])), (kp, vp, table),
                            ctx, mask, N)
    assert np.array_equal(out2, h)
    # the caller's pages are left as they were: position ctx[0] of sequence 0
    # (the block's first row) is still empty there
    assert not np.any(kp[table[0, 0], 3]) and np.any(kp2[table[0, 0], 3])
    # without the adapter, clean rows are unchanged and MASK rows differ
    no_lora, _ = forward.block(h, p, (kp, vp, table), ctx, mask, N, lora_scale=0.0)
    full, _ = forward.block(h, p, (kp, vp, table), ctx, mask, N)
    assert np.array_equal(no_lora[~mask], full[~mask]) and not np.allclose(no_lora[mask], full[mask])


def test_lm_head_statistics_are_the_row_normaliser():
    rng = np.random.default_rng(3)
    h = rng.normal(size=(3, 32))
    W = rng.normal(0, 0.3, (300, 32))
    xf, logits, stats = forward.lm_head(h, np.ones(32), W, chunk=128)
    assert stats.shape == (3, 3, 2)
    assert np.array_equal(logits, forward.bf16_round(logits))  # already bf16 values
    for i in range(3):
        M = stats[i, :, 0].max()
        S = np.sum(stats[i, :, 1] * np.exp(stats[i, :, 0] - M))
        assert abs(M - logits[i].max()) == 0
        assert abs(S - np.sum(np.exp(logits[i] - logits[i].max()))) < 1e-9

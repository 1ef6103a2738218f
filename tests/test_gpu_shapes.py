"""GPU parity on generated small shapes (hypothesis, derandomized so every run
draws the same cases): attention, the accept step along short trajectories
and the gated projections, each against the oracle with the bars of the
other GPU tests.

- attention: ragged contexts (0..600 cached tokens), odd page maps, stride
  N in 2..8 (2N block rows), 1..8 query heads per KV head, D 64 or 128,
  bf16 (2e-3 normwise per slab) or fp32 (1e-5), every split (stream-K with
  automatic or forced slices, batch-invariant chunks of 1..8 tiles), the
  block's own K/V from the pages or from its rows;
- accept: N in 2..8, vocabularies of 2..20,000 entries (ragged last chunk),
  1..8 sequences, bf16 or fp32, rows padded with NaN to a 16-byte stride,
  three steps from FRESH (so both n_draft = 0 and n_draft = N-1 occur)
  with the trajectory test's bars;
- projections: M 1..300, K a multiple of 64 up to 512, Nout 1..300, rank a
  multiple of 16 up to 128, random MASK rows: 2e-3 against the oracle and
  clean rows bit-identical to isd_linear.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import draft_verify_decoding_amd as dvd
import workload
from oracle import attention as oatt
from oracle import lora as olora

from test_gpu_accept import run_trajectory

pytestmark = pytest.mark.gpu
DEV = "cuda"
SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow],
                print_blob=True)


def to64(t):
    return t.detach().float().cpu().double().numpy()


@st.composite
def attention_cases(draw):
    C = draw(st.integers(1, 4))
    N = draw(st.integers(2, 8))
    rows = 2 * N
    Hkv = draw(st.sampled_from([1, 2, 4]))
    group = draw(st.sampled_from([g for g in (1, 2, 4, 8) if g * rows <= 128]))
    D = draw(st.sampled_from([64, 128]))
    ctx = draw(st.lists(st.integers(0, 600), min_size=C, max_size=C))
    dtype = draw(st.sampled_from(["bf16", "f32"]))
    split = draw(st.sampled_from(["auto", "forced", "invariant"]))
    slices = {"auto": 0, "forced": draw(st.integers(1, 9)),
              "invariant": dvd.attn_invariant(draw(st.integers(1, 8)))}[split]
    with_block = draw(st.booleans())
    spare = draw(st.integers(0, 5))
    seed = draw(st.integers(0, 10_000))
    return dict(C=C, rows=rows, Hq=Hkv * group, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype, slices=slices,
                with_block=with_block, spare=spare, seed=seed)


@settings(max_examples=30, **SETTINGS)
@given(attention_cases())
def test_attention_generated_shapes(p):
    print(f"generated attention case {p}", flush=True)
    dtype = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    case = workload.AttentionCase(p["seed"], C=p["C"], rows=p["rows"], Hq=p["Hq"], Hkv=p["Hkv"], D=p["D"],
                                  ctx=p["ctx"], dtype=dtype, spare_pages=p["spare"])
    kv = dvd.KVCache(case.num_pages, case.Hkv, case.D, dtype, torch.from_numpy(case.table), DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx = torch.from_numpy(case.ctx).to(DEV)
    # the pages hold the cached context, plus the block when it is read from them
    written = case.ctx if p["with_block"] else case.lengths
    dvd.isd_kv_write(kv, case.k_rows.to(DEV).contiguous(), case.v_rows.to(DEV).contiguous(),
                     torch.zeros(case.C, dtype=torch.int32, device=DEV),
                     torch.from_numpy(written.astype(np.int32)).to(DEV), dev_err=err)
    kb = vb = None
    if p["with_block"]:
        kb = torch.stack([case.k_rows[b, int(c):int(c) + case.rows] for b, c in enumerate(case.ctx)]).to(DEV)
        vb = torch.stack([case.v_rows[b, int(c):int(c) + case.rows] for b, c in enumerate(case.ctx)]).to(DEV)
        kb, vb = kb.contiguous(), vb.contiguous()
    out = dvd.isd_attention(kv, case.q.to(DEV), ctx, max_len=int(case.lengths.max()), slices=p["slices"],
                            dev_err=err, k_blk=kb, v_blk=vb)
    torch.cuda.synchronize()
    assert err.item() == 0
    kp = np.zeros((case.num_pages, 16, case.Hkv, case.D))
    vp = np.zeros_like(kp)
    oatt.kv_write(kp, vp, case.table, np.zeros(case.C, int), to64(case.k_rows), to64(case.v_rows), case.lengths)
    want = oatt.block_attention(to64(case.q), kp, vp, case.table, case.ctx)
    got = out.cpu().double().numpy()
    C, R, H, D = want.shape
    g = got.transpose(0, 2, 1, 3).reshape(C, H, R * D)
    w = want.transpose(0, 2, 1, 3).reshape(C, H, R * D)
    slab = np.abs(g - w).max(-1) / np.abs(w).max(-1)
    assert slab.max() < (2e-3 if dtype == torch.bfloat16 else 1e-5), slab.max()


@settings(max_examples=20, **SETTINGS)
@given(C=st.integers(1, 8), N=st.integers(2, 8), V=st.integers(2, 20000), bf16=st.booleans(),
       seed=st.integers(0, 10_000), sigma_q=st.sampled_from([0.2, 0.5, 1.0]))
def test_accept_generated_shapes(C, N, V, bf16, seed, sigma_q):
    print(f"generated accept case C={C} N={N} V={V} bf16={bf16} seed={seed} sigma_q={sigma_q}", flush=True)
    # rows padded (with NaN the kernels must never read) to the 16-byte row
    # alignment the call requires
    ld = (V + 7) // 8 * 8
    t, _ = run_trajectory(3, seed=seed, C=C, N=N, V=V, sigma_l=2.0, sigma_q=sigma_q,
                          dtype=torch.bfloat16 if bf16 else torch.float32, ctx0=50, ld=ld)
    assert t.compared + t.excused >= C


@settings(max_examples=20, **SETTINGS)
@given(M=st.integers(1, 300), K=st.sampled_from([64, 128, 192, 320, 512]), Nout=st.integers(1, 300),
       r=st.sampled_from([16, 32, 48, 64, 96, 128]), seed=st.integers(0, 10_000))
def test_projection_generated_shapes(M, K, Nout, r, seed):
    print(f"generated projection case M={M} K={K} Nout={Nout} r={r} seed={seed}", flush=True)
    x, W, A, B = workload.lora_case(seed, M, K, Nout, r)
    mask = np.random.default_rng(seed).random(M) < 0.5
    xd, Wd, Ad, Bd = (t.to(DEV).contiguous() for t in (x, W, A, B))
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    fused = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
    sep = base.clone()
    dvd.gated_lora_apply(xd, Ad, Bd, md, sep, scale=1.0)
    torch.cuda.synchronize()
    want = olora.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(),
                            mask, 1.0)
    for y in (fused, sep):
        got = y.cpu().double().numpy()
        assert np.abs(got - want).max() / max(np.abs(want).max(), 1e-30) < 2e-3
    clean = torch.from_numpy(~mask).to(DEV)
    assert torch.equal(fused[clean].view(torch.int32), base[clean].view(torch.int32))
    assert torch.equal(sep[clean].view(torch.int32), base[clean].view(torch.int32))
    assert torch.equal(fused.view(torch.int32), sep.view(torch.int32))

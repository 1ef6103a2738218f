"""GPU parity of the decoder-block pieces (isd_rmsnorm, isd_cast_bf16,
isd_swiglu) and of one whole chained forward (a decoder layer, the final
norm, the LM head and the accept step on its statistics) against the
oracle composed from oracle/ (oracle.forward).

Bars: a value the forward rounds to bf16 is within one bf16 rounding of the
oracle's (2^-7 relative: the fp32 and fp64 sides may round a value that
sits on a rounding boundary differently); projections and attention within
2e-3 normwise (the pages' bar, as in the other tests); chunk maxima exact,
chunk sums within 1e-5 relative; accept decisions, emitted ids and next
drafts bit-exact except on draws within 1e-5 of a boundary. Each stage is
checked on the GPU's own inputs to it (teacher forced), and the logits of
the whole chain against the oracle run from the same embeddings.
"""

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload
from draft_verify_decoding_amd import forward as gfwd
from oracle import accept as oacc
from oracle import attention as oatt
from oracle import forward as ofwd
from oracle import lora as olora
from oracle import philox

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_REL = 2.0 ** -7


def to64(t):
    return t.detach().float().cpu().double().numpy()


def within_bf16(got, want):
    """every element within one bf16 rounding of the oracle's"""
    return np.all(np.abs(got - want) <= BF16_REL * np.abs(want) + 1e-30)


def normwise(got, want):
    return np.abs(got - want).max() / np.abs(want).max()


@pytest.mark.parametrize("M,H", [(1, 4), (7, 1000), (33, 4096), (512, 4096)])
def test_rmsnorm_with_residual_add(M, H):
    print(f"rmsnorm M={M} H={H}", flush=True)
    h = workload.normal((M, H), 2.0, torch.float32, "cpu", 1, "h", M, H)
    d = workload.normal((M, H), 1.0, torch.float32, "cpu", 1, "d", M, H)
    g = workload.normal((H,), 1.0, torch.bfloat16, "cpu", 1, "g", H)
    hd = h.to(DEV)
    out = dvd.isd_rmsnorm(hd, g.to(DEV), delta=d.to(DEV))
    torch.cuda.synchronize()
    hs = h.double().numpy() + d.double().numpy()
    assert np.allclose(hd.cpu().double().numpy(), hs, rtol=1e-6, atol=1e-6)  # the residual add, in place
    want = ofwd.bf16_round(ofwd.rmsnorm(hd.cpu().double().numpy(), g.double().numpy()))
    assert within_bf16(to64(out), want)
    # without delta: h is left as it is
    h2 = hd.clone()
    out2 = dvd.isd_rmsnorm(h2, g.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(h2, hd) and torch.equal(out2.view(torch.int16), out.view(torch.int16))


def test_cast_split_and_swiglu():
    M, widths = 37, [512, 128, 128]
    src = workload.normal((M, sum(widths) + 8), 3.0, torch.float32, "cpu", 2, "src")
    outs = [torch.empty((M, w), dtype=torch.bfloat16, device=DEV) for w in widths]
    sd = src.to(DEV)
    dvd.isd_cast_bf16(sd[:, : sum(widths)], outs)  # row stride of src is sum(widths) + 8
    torch.cuda.synchronize()
    c0 = 0
    for o, w in zip(outs, widths):
        want = ofwd.bf16_round(src[:, c0:c0 + w].double().numpy())
        assert np.array_equal(to64(o), want)  # a plain rounding: the same on both sides
        c0 += w
    I = 300
    gu = workload.normal((M, 2 * I), 3.0, torch.float32, "cpu", 3, "gu")
    act = dvd.isd_swiglu(gu.to(DEV))
    torch.cuda.synchronize()
    g64 = gu.double().numpy()
    assert within_bf16(to64(act), ofwd.bf16_round(ofwd.swiglu(g64[:, :I], g64[:, I:])))


SHAPES = {
    # C, N, hidden, Hq, Hkv, D, intermediate, V, rank, contexts, weight std (W, down, LM head)
    "small": (3, 4, 256, 4, 2, 64, 512, 3000, 16, [5, 40, 100], (0.06, 0.04, 0.1)),
    # 8B-class layer: 32/8 heads of 128, hidden 4096, MLP 12,288, rank 32 (the
    # vocabulary cut to 20,000 to keep the oracle's LM head small)
    "8b": (2, 4, 4096, 32, 8, 128, 12288, 20000, 32, [300, 1100], (0.02, 0.01, 0.047)),
}


def small_forward(seed, lora, shape="small", split=False):
    """One layer, LM head and statistics through Forward. With split, Q, K
    and V carry an adapter each and run as three projections that write bf16
    q, k and v themselves; the oracle sees the same adapters stacked (A) and
    block-diagonal (B), which is the same map."""
    C, N, H, Hq, Hkv, D, I, V, r, ctx, (w_std, d_std, lm_std) = SHAPES[shape]
    R, M = 2 * N, C * 2 * N
    ctx = np.array(ctx, dtype=np.int32)
    nrm = lambda shape, std, *tag: workload.normal(shape, std, torch.bfloat16, "cpu", seed, *tag)
    nq = (Hq + 2 * Hkv) * D
    w = gfwd.LayerWeights(
        g1=workload.normal((H,), 0.1, torch.float32, "cpu", seed, "g1").add_(1.0).to(torch.bfloat16),
        g2=workload.normal((H,), 0.1, torch.float32, "cpu", seed, "g2").add_(1.0).to(torch.bfloat16),
        Wqkv=nrm((nq, H), w_std, "Wqkv"), Wo=nrm((H, Hq * D), w_std, "Wo"), Wgu=nrm((2 * I, H), w_std, "Wgu"),
        Wd=nrm((H, I), d_std, "Wd"), Aqkv=nrm((r, H), 0.05, "Aqkv"), Bqkv=nrm((nq, r), 0.05, "Bqkv"),
        Ao=nrm((r, Hq * D), 0.05, "Ao"), Bo=nrm((H, r), 0.05, "Bo"))
    gf = workload.normal((H,), 0.1, torch.float32, "cpu", seed, "gf").add_(1.0).to(torch.bfloat16)
    Wlm = nrm((V, H), lm_std, "Wlm")
    table, num_pages = workload.block_table(seed, ctx + R)
    cached_k = nrm((C, int(ctx.max()), Hkv, D), 1.0, "ck")
    cached_v = nrm((C, int(ctx.max()), Hkv, D), 1.0, "cv")
    kv = dvd.KVCache(num_pages, Hkv, D, torch.bfloat16, torch.from_numpy(table), DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write(kv, cached_k.to(DEV), cached_v.to(DEV), torch.zeros(C, dtype=torch.int32, device=DEV),
                     torch.from_numpy(ctx).to(DEV), dev_err=err)
    mask = workload.stride_mask(M, N)
    dev = lambda t: None if t is None else t.to(DEV).contiguous()
    wd = gfwd.LayerWeights(*(dev(getattr(w, k)) for k in ("g1", "g2", "Wqkv", "Wo", "Wgu", "Wd", "Aqkv", "Bqkv", "Ao",
                                                           "Bo")))
    if split:
        widths = (Hq * D, Hkv * D, Hkv * D)
        ads = [(nrm((r, H), 0.05, "Asplit", j), nrm((n, r), 0.05, "Bsplit", j)) for j, n in enumerate(widths)]
        wd.qkv_adapters = [(dev(a), dev(b)) for a, b in ads]
        wd.Aqkv = wd.Bqkv = None
        w.Aqkv = torch.cat([a for a, _ in ads])
        w.Bqkv = torch.block_diag(*[b.float() for _, b in ads]).to(torch.bfloat16)
    k_all = torch.empty((1, C, R, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v_all = torch.empty_like(k_all)
    fw = gfwd.Forward([wd], [kv], torch.from_numpy(ctx).to(DEV), torch.from_numpy(mask.astype(np.uint8)).to(DEV),
                      gf.to(DEV), Wlm.to(DEV), C, N, Hq, Hkv, D, int(ctx.max()) + R, dvd.attn_invariant(2), k_all,
                      v_all, lora=lora, dev_err=err)
    h0 = workload.normal((M, H), 1.0, torch.float32, "cpu", seed, "h0")
    fw(h0.to(DEV))
    torch.cuda.synchronize()
    assert err.item() == 0
    p = {k: (getattr(w, k).double().numpy()) for k in ("g1", "g2", "Wqkv", "Wo", "Wgu", "Wd", "Aqkv", "Bqkv", "Ao",
                                                         "Bo")}
    p.update(Hq=Hq, Hkv=Hkv, D=D)
    kp = np.zeros((num_pages, 16, Hkv, D))
    vp = np.zeros_like(kp)
    oatt.kv_write(kp, vp, table, np.zeros(C, int), to64(cached_k), to64(cached_v), ctx)
    return dict(fw=fw, p=p, kv=(kp, vp, table), ctx=ctx, mask=mask, h0=h0.double().numpy(), gf=gf.double().numpy(),
                Wlm=Wlm.double().numpy(), k_all=k_all, v_all=v_all, C=C, N=N, R=R, M=M, V=V, Hq=Hq, Hkv=Hkv, D=D,
                lora=lora, split=split)


@pytest.mark.parametrize("lora,shape,split", [("gated", "small", False), ("off", "small", False),
                                              ("gated", "8b", False), ("gated", "8b", True), ("off", "small", True)])
def test_one_chained_layer_lm_head_and_accept_against_the_oracle(lora, shape, split):
    """One decoder layer chained through its real outputs, the LM head and
    the accept on its statistics, stage by stage (each stage on the GPU's own
    input to it) and end to end against the oracle's chain. The 8B-class
    layer runs its 16 rows through the few-row projection kernel; split runs
    Q, K and V as three projections with their own adapters."""
    print(f"chained forward, lora {lora}, shape {shape}, split {split}", flush=True)
    s = small_forward(21, lora, shape, split)
    fw, p, C, N, R, M = s["fw"], s["p"], s["C"], s["N"], s["R"], s["M"]
    scale = 1.0 if lora == "gated" else 0.0
    mask = s["mask"]
    # stage by stage, each on the GPU's own input to it
    x = to64(fw.x)
    assert within_bf16(x, ofwd.bf16_round(ofwd.rmsnorm(s["h0"], p["g1"])))
    yqkv = olora.gated_lora(x, p["Wqkv"], p["Aqkv"], p["Bqkv"], mask, scale)
    qw, kw = s["Hq"] * s["D"], s["Hkv"] * s["D"]
    q, k, v = (to64(t).reshape(M, -1) for t in (fw.q, s["k_all"][0], s["v_all"][0]))
    if split:  # bf16 outputs of the projections: fp32 tolerance plus one rounding
        for got, want in ((q, yqkv[:, :qw]), (k, yqkv[:, qw:qw + kw]), (v, yqkv[:, qw + kw:])):
            assert normwise(got, want) < 2e-3 + 2.0 ** -8
    else:
        assert normwise(to64(fw.yqkv), yqkv) < 2e-3
        y = to64(fw.yqkv)
        assert np.array_equal(q, ofwd.bf16_round(y[:, :qw]))
        assert np.array_equal(k, ofwd.bf16_round(y[:, qw:qw + kw]))
        assert np.array_equal(v, ofwd.bf16_round(y[:, qw + kw:]))
    kp, vp, table = (a.copy() for a in s["kv"])
    oatt.kv_write(kp, vp, table, s["ctx"], to64(s["k_all"][0]), to64(s["v_all"][0]), np.full(C, R))
    att = oatt.block_attention(to64(fw.q), kp, vp, table, s["ctx"])
    ob = to64(fw.ob).reshape(att.shape)
    for b in range(C):
        for hq in range(s["Hq"]):  # fp32 tolerance plus the output's bf16 rounding
            assert normwise(ob[b, :, hq], att[b, :, hq]) < 2e-3 + 2.0 ** -8
    yo = olora.gated_lora(to64(fw.ob), p["Wo"], p["Ao"], p["Bo"], mask, scale)
    assert normwise(to64(fw.yo), yo) < 2e-3
    h1 = s["h0"] + to64(fw.yo)
    assert within_bf16(to64(fw.x2), ofwd.bf16_round(ofwd.rmsnorm(h1, p["g2"])))
    assert normwise(to64(fw.gu), olora.linear(to64(fw.x2), p["Wgu"])) < 2e-3
    g = to64(fw.gu)
    I = g.shape[1] // 2
    assert within_bf16(to64(fw.act), ofwd.bf16_round(ofwd.swiglu(g[:, :I], g[:, I:])))
    assert normwise(to64(fw.yd), olora.linear(to64(fw.act), p["Wd"])) < 2e-3
    h2 = h1 + to64(fw.yd)
    assert np.allclose(to64(fw.h), h2, rtol=1e-5, atol=1e-5)
    assert within_bf16(to64(fw.xf), ofwd.bf16_round(ofwd.rmsnorm(to64(fw.h), s["gf"])))
    logits = to64(fw.logits).reshape(M, -1)
    # bf16 logits within one rounding (2^-8 relative) of the exact product of
    # the GPU's own normalised rows, plus the fp32 accumulation error over K
    # (1e-5 of the row block's largest logit), as in the LM-head tests
    exact = olora.linear(to64(fw.xf), s["Wlm"])
    assert np.all(np.abs(logits - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-5 * np.abs(exact).max())
    st = to64(fw.stats).reshape(M, -1, 2)
    for m in range(M):
        want = oacc.chunk_stats(logits[m], 8192)
        assert np.array_equal(st[m, :, 0], want[:, 0])
        assert np.all(np.abs(st[m, :, 1] / want[:, 1] - 1) <= 1e-5)
    # the whole chain from the same embeddings, oracle all the way
    o_h, _ = ofwd.block(s["h0"], p, s["kv"], s["ctx"], mask, N, lora_scale=scale)
    _, o_logits, _ = ofwd.lm_head(o_h, s["gf"], s["Wlm"])
    e2e = normwise(logits, o_logits)
    print(f"end-to-end logits, normwise error {e2e:.2e}", flush=True)
    assert e2e < 1e-2
    # the accept step on these logits, with the LM head's statistics, against
    # the oracle on the same logits (a FRESH step: bonus and proposals)
    st_in, st_out = dvd.SeqState(C, N), dvd.SeqState(C, N)
    out = dvd.isd_accept(fw.logits, None, st_in, st_out, N, 5, 0, V=s["V"], diag=True, chunk_stats=fw.stats)
    torch.cuda.synchronize()
    o = oacc.accept_step(logits.reshape(C, R, -1), None, np.zeros(C, np.int64), np.full((C, N - 1), -1, np.int64),
                         np.zeros(C, np.int64), philox.step_uniforms(5, 0, C, N), N)
    flags = oacc.flagged(o, 1e-5)
    for b in range(C):
        if flags[b]:
            continue
        assert np.array_equal(out.emit.cpu().numpy()[b], o["emit"][b])
        assert np.array_equal(st_out.drafts.cpu().numpy()[b], o["drafts_next"][b])
        assert np.all(np.abs(st_out.q_x.cpu().numpy()[b] - o["q_x_next"][b]) <= 1e-5)

"""Throughput of the ISD step on one MI355X.

Workload (stationary batch, 8B-class shapes): C = 64 sequences, stride N = 4
(8-row blocks: 4 verify + 4 MASK), 36 layers of grouped-query attention with
32 query heads, 8 KV heads, head_dim 128, bf16 paged KV cache in 16-token
pages placed by a seeded shuffle, cached contexts drawn uniformly from
1024..8192 per sequence, vocabulary 151,936 with draft noise set for a mean
acceptance of 0.9, gated-LoRA (rank 32 per projection) Q/K/V/O projections
on the 512 block rows of each layer (Q, K and V fused into one 6144-wide
projection). All inputs are seeded synthetic tensors (no weights or
datasets exist for this), resident in HBM before the timed region.

One step = for each of the 36 layers: gated fused QKV projection, KV write of
the block, block attention over the pages, gated O projection; then the
accept step over the block logits (verify, residual / bonus draw, proposals,
KV commit). The MLP and the LM head are not part of the library; the logits
the LM head would produce are synthetic and pre-generated per step.

--workload 32b runs the same step at 32B-class shapes instead: C = 16
sequences of 16,384 cached tokens, 64 layers of 64 query / 8 KV heads,
head_dim 128, hidden 5120 (Q|K|V 10240 wide, O from 8192 to 5120), with the
stride (--N) and the acceptance (--accept) of one cell of the stride sweep.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                       [--workload 8b|32b] [--N N] [--accept P]
Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ISD accepted tokens/s at C=64,N=4 (8B shapes); attn+accept HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
PROBE_EVERY = 8  # timed steps between the ones bracketed with HIP events

CFG = dict(C=64, N=4, Hq=32, Hkv=8, D=128, layers=36, V=151936, hidden=4096, intermediate=12288, lora_rank=32,
           ctx=("uniform", 1024, 8192), accept=0.9, sigma_l=3.0, seed=3, proposal="sample")
CFG_32B = dict(CFG, C=16, Hq=64, Hkv=8, D=128, layers=64, hidden=5120, intermediate=25600, ctx=16384)
CFG_8B1 = dict(CFG, C=1, ctx=4096)  # the single-sequence 8B step


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_bytes(ctx, cfg):
    """Algorithmic HBM bytes of one isd_attention call: every K and V element
    of positions 0..ctx_b + 2N - 1 once (bf16), the queries (bf16) and the
    fp32 outputs."""
    R = 2 * cfg["N"]
    kv = int(np.sum(ctx + R)) * cfg["Hkv"] * cfg["D"] * 2 * 2
    q = cfg["C"] * R * cfg["Hq"] * cfg["D"] * 2
    o = cfg["C"] * R * cfg["Hq"] * cfg["D"] * 4
    return kv + q + o


def accept_bytes(n_draft, accepted, cfg):
    """Algorithmic HBM bytes of one accept step: each logits row the step
    reads once (rows 0..n+N-1 per sequence, bf16), plus the two rows of the
    residual (P_a and the old Q_{a+1}) for sequences that rejected a draft."""
    V, N = cfg["V"], cfg["N"]
    rows = int(np.sum(n_draft + N))
    resid = int(np.sum(accepted < n_draft)) * 2
    return (rows + resid) * V * 2


def projection_flops(cfg):
    """Algorithmic flops of the two projections of one layer: the base
    product over all 2N*C rows plus, when the LoRA is on, the rank-r delta
    (x A^T then U B^T) on the N*C MASK rows."""
    C, N, H, r = cfg["C"], cfg["N"], cfg["hidden"], cfg["lora_rank"]
    M, Mm = C * 2 * N, C * N
    n_qkv = (cfg["Hq"] + 2 * cfg["Hkv"]) * cfg["D"]
    n_att = cfg["Hq"] * cfg["D"]  # width of the attention output (input of O)
    lora = cfg.get("lora", "gated") == "gated"
    qkv = 2 * M * H * n_qkv + lora * 2 * Mm * r * (3 * H + n_qkv)  # three A [r, H]; B rows sum to n_qkv
    o = 2 * M * n_att * H + lora * 2 * Mm * r * (n_att + H)
    return qkv, o


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_hbm_traffic_c64_n4.txt")  # default workload only
KERNEL_SOURCES = [os.path.join(ROOT, "draft_verify_decoding_amd", "csrc", f)
                  for f in ("isd_attention.hip", "isd_common.hpp")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per isd_attention call from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, or None when the attention source has changed
    since they were taken (or they are missing)."""
    try:
        lines = [l for l in open(TRAFFIC_FILE) if l.startswith("RESULT ")]
        rec = json.loads(lines[-1][len("RESULT "):])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def counter_means(root):
    """{(kernel, counter): [values per dispatch]} from a rocprofv3 --pmc CSV
    output tree."""
    import collections
    import csv
    acc = collections.defaultdict(list)
    for dirpath, _, files in os.walk(root):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, f)) as fh:
                    for row in csv.DictReader(fh):
                        acc[(row["Kernel_Name"], row["Counter_Name"])].append(float(row["Counter_Value"]))
    return acc


def short_kernel(name):
    name = name.split("(")[0].replace("unsigned short", "bf16")
    return name[5:] if name.startswith("void ") else name


def traffic_report(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, algo_json):
    """HBM bytes per dispatch of the step's kernels from FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter
    reads for a plain 1 GiB device copy, against the algorithmic bytes the
    profiled run recorded (--algo-out). Prints a markdown report ending in a
    RESULT line for the attention call."""
    fetch, write = counter_means(fetch_dir), counter_means(write_dir)
    cf, cw = counter_means(copy_fetch_dir), counter_means(copy_write_dir)
    algo = json.load(open(algo_json))
    copied_kib = algo["copy_probe_bytes"] / 1024

    def copy_factor(acc, counter):
        vals = [v for (k, c), vs in acc.items() if c == counter and "copy" in k.lower() for v in vs]
        return copied_kib / (sum(vals) / len(vals))

    ff, fw = copy_factor(cf, "FETCH_SIZE"), copy_factor(cw, "WRITE_SIZE")
    print(f"- FETCH_SIZE scale: {ff:.5f} (a 1 GiB copy reads {copied_kib / ff:.0f} KiB)")
    print(f"- WRITE_SIZE scale: {fw:.5f} (a 1 GiB copy writes {copied_kib / fw:.0f} KiB)\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) |")
    print("|---|---|---|---|---|")
    per = {}
    for (k, c), vs in sorted(fetch.items()):
        if c != "FETCH_SIZE":
            continue
        wv = write.get((k, "WRITE_SIZE"), [0.0])
        f_kib, w_kib = sum(vs) / len(vs), sum(wv) / len(wv)
        mb = (f_kib * ff + w_kib * fw) * 1024 / 1e6
        per[short_kernel(k)] = (len(vs), f_kib, w_kib, mb)
        print(f"| `{short_kernel(k)}` | {len(vs)} | {f_kib:.1f} | {w_kib:.1f} | {mb:.2f} |")
    att = [v for k, v in per.items() if k.startswith("isd::attention_kernel") or k.startswith("isd::attention_merge")]
    call_bytes = sum(v[3] for v in att) * 1e6
    algo_call = float(np.mean(algo["attention_bytes_per_step"]))
    print(f"\n- isd_attention call (main + merge): {call_bytes / 1e9:.4f} GB per call; algorithmic "
          f"{algo_call / 1e9:.4f} GB (ratio {call_bytes / algo_call:.4f})")
    acc_k = [v for k, v in per.items() if k.startswith("isd::accept_")]
    if acc_k:
        acc_bytes = sum(v[3] for v in acc_k) * 1e6
        algo_acc = float(np.mean(algo["accept_bytes_per_step"]))
        print(f"- isd_accept step: {acc_bytes / 1e6:.1f} MB per step; algorithmic {algo_acc / 1e6:.1f} MB "
              f"(ratio {acc_bytes / algo_acc:.4f})")
    rec = {"kernel_source_sha256": kernel_source_hash(), "hbm_bytes_per_call": int(call_bytes),
           "algorithmic_bytes_per_call": int(algo_call), "ratio_to_algorithmic": round(call_bytes / algo_call, 4)}
    print("\nRESULT " + json.dumps(rec))


def summarize_counters(root):
    """Per-kernel mean of every counter in a rocprofv3 --pmc CSV output tree
    (KiB per dispatch for FETCH_SIZE / WRITE_SIZE), one line per kernel and
    counter."""
    for (k, c), v in sorted(counter_means(root).items()):
        print(f"{c:28s} dispatches={len(v):5d} mean={sum(v) / len(v):.6g}  {k[:90]}")


def build(cfg, steps_total, dev):
    import draft_verify_decoding_amd as dvd
    import workload

    C, N, Hq, Hkv, D, L = cfg["C"], cfg["N"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["layers"]
    R = 2 * N
    seed = cfg["seed"]
    ctx0 = workload.contexts(seed, C, cfg["ctx"])
    capacity = ctx0 + R + steps_total * N + 16
    table, num_pages = workload.block_table(seed, capacity)
    table_t = torch.from_numpy(table)
    log(f"[bench] {L} layers x {num_pages} pages; KV pool {2 * L * num_pages * Hkv * D * 16 * 2 / 1e9:.1f} GB")

    # KV pools: fill every layer from one random source (values do not
    # change the work; every layer still lives in its own HBM pages)
    per_pool = num_pages * Hkv * D * 16
    src = workload.normal((per_pool,), 1.0, torch.bfloat16, dev, seed, "kv-src")
    # one allocation for all layers (shared block table), so a step's KV
    # commit is one isd_kv_write_layers launch
    kvs, layer_stride = dvd.KVCache.stacked(L, num_pages, Hkv, D, torch.bfloat16, table_t, dev)
    for kv in kvs:
        kv.k_pages.copy_(src)
        kv.v_pages.copy_(src.flip(0))
    del src

    M, H, r = C * R, cfg["hidden"], cfg["lora_rank"]
    HD = Hq * D  # attention output width, the O projection's input
    mask = torch.from_numpy(workload.stride_mask(M, N).astype(np.uint8)).to(dev)
    # the block's K/V rows of every layer, stacked for the commit
    k_all = torch.stack([workload.normal((C, R, Hkv, D), 1.0, torch.bfloat16, dev, seed, "kb", l) for l in range(L)])
    v_all = torch.stack([workload.normal((C, R, Hkv, D), 1.0, torch.bfloat16, dev, seed, "vb", l) for l in range(L)])
    layers = []
    for l in range(L):
        lay = dict(
            q=workload.normal((C, R, Hq, D), 1.0, torch.bfloat16, dev, seed, "q", l),
            k=k_all[l],
            v=v_all[l],
            x=workload.normal((M, H), 1.0, torch.bfloat16, dev, seed, "x", l),
            xo=workload.normal((M, HD), 1.0, torch.bfloat16, dev, seed, "xo", l),
            out=torch.empty((C, R, Hq, D), dtype=torch.float32, device=dev),
        )
        # Q, K and V run as one projection (weights stacked, 6144 outputs);
        # their three rank-r adapters stack into A [3r, H] and a block-
        # diagonal B [6144, 3r], which is the same delta on each slice.
        proj = {}
        parts = [("q", Hq * D), ("k", Hkv * D), ("v", Hkv * D)]
        Ws, As, Bs = [], [], []
        for name, nout in parts:
            Ws.append(workload.normal((nout, H), 0.02, torch.bfloat16, dev, seed, "W", name, l))
            As.append(workload.normal((r, H), 0.01, torch.bfloat16, dev, seed, "A", name, l))
            Bs.append(workload.normal((nout, r), 0.01, torch.bfloat16, dev, seed, "B", name, l))
        n_qkv = sum(n for _, n in parts)
        Bqkv = torch.zeros((n_qkv, 3 * r), dtype=torch.bfloat16, device=dev)
        off = 0
        for i, (_, nout) in enumerate(parts):
            Bqkv[off:off + nout, i * r:(i + 1) * r] = Bs[i]
            off += nout
        proj["qkv"] = dict(W=torch.cat(Ws).contiguous(), A=torch.cat(As).contiguous(), B=Bqkv,
                           y=torch.empty((M, n_qkv), dtype=torch.float32, device=dev))
        proj["o"] = dict(W=workload.normal((H, HD), 0.02, torch.bfloat16, dev, seed, "W", "o", l),
                         A=workload.normal((r, HD), 0.01, torch.bfloat16, dev, seed, "A", "o", l),
                         B=workload.normal((H, r), 0.01, torch.bfloat16, dev, seed, "B", "o", l),
                         y=torch.empty((M, H), dtype=torch.float32, device=dev))
        lay["proj"] = proj
        layers.append(lay)
    lora_ws = dvd.lora_workspace(M, 3 * r, dev)
    return dict(ctx0=ctx0, kvs=kvs, layer_stride=layer_stride, k_all=k_all, v_all=v_all, layers=layers, mask=mask,
                lora_ws=lora_ws, table=table)


def dry_run(cfg, steps_total, ctx0, dev):
    """Accept-only pass that fixes the trajectory: the logits of every step
    (drawn from the synthetic teacher given the state) are kept in HBM, with
    the per-step contexts, draft counts and accepted lengths."""
    import draft_verify_decoding_amd as dvd
    import workload

    C, N, V = cfg["C"], cfg["N"], cfg["V"]
    R = 2 * N
    sigma_q = workload.SIGMA_Q_V151936[cfg["accept"]]
    teacher = workload.TeacherLogits(cfg["seed"], C, V, steps_total * N + R + 1, cfg["sigma_l"], sigma_q,
                                     torch.bfloat16, dev)
    ctx0_t = torch.from_numpy(ctx0.astype(np.int64)).to(dev)
    ctx = torch.from_numpy(ctx0.astype(np.int32)).to(dev)
    s_in, s_out = dvd.SeqState(C, N, dev), dvd.SeqState(C, N, dev)
    ws = dvd.accept_workspace(C, N, V, R, device=dev)
    logits, ctxs, nds, accs = [], [], [], []
    prev = None
    for t in range(steps_total):
        lg = teacher.block(t, ctx.long(), ctx0_t, s_in.n_draft.long(), R).contiguous()
        ctxs.append(ctx.cpu().numpy().copy())
        nds.append(s_in.n_draft.cpu().numpy().copy())
        out = dvd.isd_accept(lg, prev, s_in, s_out, N, cfg["seed"], t, ws=ws, ctx=ctx, proposal=cfg["proposal"])
        accs.append(out.accepted.cpu().numpy().copy())
        logits.append(lg)
        prev = lg
        s_in, s_out = s_out, s_in
    final_ctx = ctx.cpu().numpy().copy()
    del teacher
    torch.cuda.synchronize()
    return logits, np.array(ctxs), np.array(nds), np.array(accs), final_ctx


def lm_head_leg(cfg, dev, calls=20):
    """isd_lm_head at the step's shape (C*2N rows, hidden, vocabulary) on
    seeded random weights, timed with HIP events after the timed steps; and
    isd_accept on its logits (FRESH state) with and without the chunk
    statistics it produced, which is the statistics pass the LM head saves.
    The step itself keeps the teacher's logits: random weights cannot give
    the calibrated acceptance."""
    import draft_verify_decoding_amd as dvd
    import workload

    C, N, H, V = cfg["C"], cfg["N"], cfg["hidden"], cfg["V"]
    M = C * 2 * N
    W = workload.normal((V, H), 3.0 / H ** 0.5, torch.bfloat16, dev, cfg["seed"], "lm-W")
    h = workload.normal((M, H), 1.0, torch.bfloat16, dev, cfg["seed"], "lm-h")
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    nch = (V + 8191) // 8192
    stats = torch.empty((M, nch, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(dvd.isd_lm_head_workspace_size(M, V), dtype=torch.uint8, device=dev)
    call = dvd.prepare_lm_head(h, W, logits, stats, ws)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    us = timed(call, calls)
    s_in, s_out = dvd.SeqState(C, N, dev), dvd.SeqState(C, N, dev)
    acc_ws = dvd.accept_workspace(C, N, V, 2 * N, device=dev)
    acc_out = dvd.AcceptOutputs(C, N, 2 * N, dev, diag=False)
    lg3, st3 = logits.view(C, 2 * N, V), stats.view(C, 2 * N, nch, 2)
    own = timed(lambda: dvd.isd_accept(lg3, None, s_in, s_out, N, cfg["seed"], 0, out=acc_out, ws=acc_ws), calls)
    given = timed(lambda: dvd.isd_accept(lg3, None, s_in, s_out, N, cfg["seed"], 0, out=acc_out, ws=acc_ws,
                                         chunk_stats=st3), calls)
    flops = 2.0 * M * H * V
    wbytes = V * H * 2
    res = {"shape": f"{M} x {H} -> {V}", "us_per_call": round(us, 2),
           "achieved_tflops": round(flops / us / 1e6, 1), "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
           "weight_gbps": round(wbytes / us / 1e3, 1),
           "accept_fresh_us_own_stats": round(own, 2), "accept_fresh_us_lm_head_stats": round(given, 2)}
    del W, h, logits, stats, ws
    return res


def forward_leg(cfg, st, dev, slices, steps=6, warmup=2):
    """The whole synthetic forward of the step, chained through its real
    outputs: for every layer RMSNorm, gated Q|K|V projection, bf16 q/k/v,
    attention of the block over the pages, gated O projection, residual add
    and RMSNorm, gate|up projection, SwiGLU, down projection; then the final
    norm, the LM head (logits and their chunk statistics), isd_accept on
    those statistics, the KV commit of the accepted rows and the next
    block's assembly. Random weights of the 8B-class shapes (intermediate
    12288); the block's embeddings are a fixed random input. Timed with the
    adapters at rank 32 (stacked on the fused Q|K|V) and at rank 128 (one
    per projection, Q, K and V then run as three projections), each against
    the same forward with the base projections only: alpha is the ratio of
    the step times (the pages quote 1.12 at rank 128)."""
    import draft_verify_decoding_amd as dvd
    import workload
    from draft_verify_decoding_amd import forward as fwd

    C, N, Hq, Hkv, D, L, V, H = (cfg[k] for k in ("C", "N", "Hq", "Hkv", "D", "layers", "V", "hidden"))
    I = cfg["intermediate"]
    R, M, seed = 2 * N, cfg["C"] * 2 * cfg["N"], cfg["seed"]
    nq = (Hq + 2 * Hkv) * D
    nrm = lambda shape, std, *tag: workload.normal(shape, std, torch.bfloat16, dev, seed, "fwd", *tag)
    ones = torch.ones(H, dtype=torch.bfloat16, device=dev)
    t0 = time.perf_counter()
    base = [dict(Wqkv=nrm((nq, H), 0.02, "Wqkv", l), Wo=nrm((H, Hq * D), 0.02, "Wo", l),
                 Wgu=nrm((2 * I, H), 0.02, "Wgu", l), Wd=nrm((H, I), 0.02, "Wd", l)) for l in range(L)]

    def stacked(l, r):
        A = nrm((3 * r, H), 0.01, "Aqkv", r, l)
        B = torch.zeros((nq, 3 * r), dtype=torch.bfloat16, device=dev)
        off = 0
        for i, w in enumerate((Hq * D, Hkv * D, Hkv * D)):
            B[off:off + w, i * r:(i + 1) * r] = nrm((w, r), 0.01, "Bqkv", r, i, l)
            off += w
        return A, B

    def layers(r, split):
        out = []
        for l, b in enumerate(base):
            kw = dict(Ao=nrm((r, Hq * D), 0.01, "Ao", r, l), Bo=nrm((H, r), 0.01, "Bo", r, l))
            if split:
                kw["qkv_adapters"] = [(nrm((r, H), 0.01, "Aq", r, i, l), nrm((w, r), 0.01, "Bq", r, i, l))
                                      for i, w in enumerate((Hq * D, Hkv * D, Hkv * D))]
            else:
                kw["Aqkv"], kw["Bqkv"] = stacked(l, r)
            out.append(fwd.LayerWeights(ones, ones, b["Wqkv"], b["Wo"], b["Wgu"], b["Wd"], **kw))
        return out

    Wlm = nrm((V, H), 3.0 / H ** 0.5, "Wlm")
    h0 = workload.normal((M, H), 1.0, torch.float32, dev, seed, "fwd-h0")
    mask = st["mask"]
    ctx0 = torch.from_numpy(st["ctx0"].astype(np.int32)).to(dev)
    max_len = int(st["ctx0"].max()) + R + (steps + warmup + 1) * N
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    log(f"[bench] forward leg: weights built in {time.perf_counter() - t0:.1f} s")

    def run(lw, lora):
        ctx = ctx0.clone()
        ctx_prev = torch.empty_like(ctx)
        fw = fwd.Forward(lw, st["kvs"], ctx, mask, ones, Wlm, C, N, Hq, Hkv, D, max_len, slices, st["k_all"],
                         st["v_all"], lora=lora, dev_err=err, dev=dev)
        s = [dvd.SeqState(C, N, dev), dvd.SeqState(C, N, dev)]
        out = dvd.AcceptOutputs(C, N, R, dev, diag=False)
        ws = dvd.accept_workspace(C, N, V, R, device=dev)
        acc = [dvd.prepare_accept(fw.logits_buf[par], fw.logits_buf[1 - par], s[par], s[1 - par], N, seed, out, ws,
                                  ctx=ctx, dev_err=err, chunk_stats=fw.stats) for par in (0, 1)]
        commit = dvd.prepare_kv_write_layers(st["kvs"][0], st["layer_stride"], st["k_all"], st["v_all"], ctx_prev,
                                             out.kv_commit, dev_err=err)
        tok = torch.empty((C, R), dtype=torch.int32, device=dev)
        tokens = 0

        def one(t):
            par = t % 2
            ctx_prev.copy_(ctx)
            fw(h0, par)
            acc[par](t)
            commit()
            dvd.isd_block_assemble(s[1 - par], out.emit, out.n_emit, ctx, N, V, tokens=tok, dev_err=err)

        for t in range(warmup):
            one(t)
        torch.cuda.synchronize()
        c0 = ctx.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warmup, warmup + steps):
            one(t)
        e1.record()
        torch.cuda.synchronize()
        assert err.item() == 0, f"device error flags {err.item()}"
        tokens = int((ctx - c0).sum())
        ms = e0.elapsed_time(e1) / steps
        del fw, acc, commit
        return ms, tokens

    res = {}
    for name, r, split, lora in (("rank32", 32, False, "gated"), ("base_fused", 32, False, "off"),
                                 ("rank128", 128, True, "gated"), ("base_split", 128, True, "off")):
        lw = layers(r, split)
        ms, tokens = run(lw, lora)
        del lw
        res[name] = (ms, tokens)
        log(f"[bench] forward {name}: {ms:.3f} ms per step, {tokens} tokens in {steps} steps")
    out = {
        "workload": (f"whole forward of the step: {L} layers (RMSNorm, gated Q|K|V, attention, gated O, RMSNorm, "
                     f"SwiGLU MLP {H}->{2 * I}->{H}), final norm, LM head {H}->{V} with chunk statistics, accept, "
                     "KV commit, block assembly; random weights"),
        "ms_per_step": {k: round(v[0], 3) for k, v in res.items()},
        "tokens_per_s": {k: round(v[1] / (v[0] * steps / 1e3), 1) for k, v in res.items()},
        "alpha": {"rank32": round(res["rank32"][0] / res["base_fused"][0], 4),
                  "rank128": round(res["rank128"][0] / res["base_split"][0], 4)},
        "alpha_pages": 1.12,
        "steps": steps,
        "note": ("random weights give flat, unrelated p and q rows, so few drafts pass: the tokens per step here "
                 "are not the calibrated workload's; alpha is a ratio of step times on the same trajectory shape"),
    }
    return out


def cpu_baseline(cfg, fwd_seqs=8, accept_seqs=48, accept_steps=14, layers_timed=None):
    """The oracle, as it stands, on a bounded sample of the same workload
    (about 10 s on 16 host cores): (a) block attention + gated Q/K/V/O
    projections of every layer (or of the first `layers_timed`, scaled to
    all of them) for `fwd_seqs` sequences with contexts drawn from the
    workload's distribution; (b) the accept step for `accept_seqs` sequences
    over `accept_steps` steps from FRESH at the full vocabulary. Returns
    tokens/s of one sequence-step (forward + accept) scaled by the tokens it
    emits."""
    import workload
    from oracle import accept as oacc
    from oracle import attention as oatt
    from oracle import lora as olora
    from oracle import philox

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    C, N, Hq, Hkv, D, V = cfg["C"], cfg["N"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["V"]
    R, H, r = 2 * N, cfg["hidden"], cfg["lora_rank"]
    ctxs = workload.contexts(cfg["seed"], max(C, fwd_seqs), cfg["ctx"])[:fwd_seqs]
    L = cfg["layers"]
    Lt = layers_timed or L

    t_fwd = 0.0
    for l in range(Lt * fwd_seqs):
        case = workload.AttentionCase(cfg["seed"] + 100 + l, C=1, rows=R, Hq=Hq, Hkv=Hkv, D=D,
                                      ctx=int(ctxs[l % fwd_seqs]))
        kp = np.zeros((case.num_pages, 16, Hkv, D))
        vp = np.zeros_like(kp)
        oatt.kv_write(kp, vp, case.table, [0], case.k_rows.double().numpy(), case.v_rows.double().numpy(),
                      case.lengths)
        q = case.q.double().numpy()
        mats = []
        for name, kin, nout in (("q", H, Hq * D), ("k", H, Hkv * D), ("v", H, Hkv * D), ("o", Hq * D, H)):
            x, W, A, B = (t.double().numpy() for t in workload.lora_case(cfg["seed"] + l // fwd_seqs, R, kin, nout, r))
            mats.append((x, W, A, B))
        mask = workload.stride_mask(R, N)
        t0 = time.perf_counter()
        oatt.block_attention(q, kp, vp, case.table, case.ctx)
        for x, W, A, B in mats:
            olora.gated_lora(x, W, A, B, mask, 1.0)
        t_fwd += time.perf_counter() - t0
    t_fwd_seq_step = t_fwd / fwd_seqs * L / Lt

    sigma_q = workload.SIGMA_Q_V151936[cfg["accept"]]
    teacher = workload.TeacherLogits(cfg["seed"], accept_seqs, V, accept_steps * N + R + 1, cfg["sigma_l"],
                                     sigma_q, torch.bfloat16, "cpu")
    ctx0 = torch.zeros(accept_seqs, dtype=torch.int64)
    ctx = ctx0.clone()
    n = np.zeros(accept_seqs, np.int64)
    drafts = np.full((accept_seqs, N - 1), -1, np.int64)
    qrow = np.zeros(accept_seqs, np.int64)
    prev = None
    tokens = 0
    t_acc = 0.0
    for t in range(accept_steps):
        lg = teacher.block(t, ctx, ctx0, torch.from_numpy(n), R).double().numpy()
        u = philox.step_uniforms(cfg["seed"], t, accept_seqs, N)
        t0 = time.perf_counter()
        o = oacc.accept_step(lg, prev, n, drafts, qrow, u, N)
        t_acc += time.perf_counter() - t0
        tokens += int(o["n_emit"].sum())
        ctx += torch.from_numpy(o["kv_commit"])
        n, drafts, qrow, prev = o["n_draft_next"], o["drafts_next"], o["q_row_next"], lg
    seq_steps = accept_seqs * accept_steps
    t_step = t_fwd_seq_step + t_acc / seq_steps
    tok_per_seq_step = tokens / seq_steps
    value = tok_per_seq_step / t_step
    ctx_note = f"contexts {int(ctxs.min())}..{int(ctxs.max())}" if ctxs.min() != ctxs.max() else f"context {int(ctxs[0])}"
    layer_note = f"all {L} layers" if Lt == L else f"{Lt} of {L} layers timed and scaled to {L}"
    sample = (f"oracle (numpy fp64): attention + gated Q/K/V/O projections, {layer_note}, of "
              f"{fwd_seqs} sequences ({ctx_note}), "
              f"{t_fwd_seq_step:.2f} s per sequence-step; accept for {accept_seqs} sequences x "
              f"{accept_steps} steps from FRESH at V={V}, {t_acc / seq_steps * 1e3:.1f} ms per "
              f"sequence-step, {tok_per_seq_step:.3f} tokens per sequence-step; "
              f"{t_fwd + t_acc:.1f} s of timed CPU work")
    # cores: the threads the oracle's BLAS actually ran with; beside it the
    # host's cores as the process sees them (affinity) and as the OS counts them
    return dict(value=value, unit="tokens/s", cores=int(cores), kind="oracle", sample=sample,
                host_cores_affinity=len(os.sched_getaffinity(0)), host_cores_os=os.cpu_count())


def read_probe():
    """HBM rates that plain vendor kernels reach on this GPU: torch's sum of
    a 4 GiB bf16 tensor (fp32 accumulation: reads 4 GiB, writes 4 bytes), the
    vendor BLAS matrix-vector product over the same 4 GiB as a 65536 x 32768
    matrix, and a 1 GiB device copy (reads and writes 1 GiB), each timed on
    HIP events over 10 calls after 3 warmup calls, on the stream the kernels
    run on."""
    torch.cuda.set_device(0)
    n = 1 << 31
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    out = {}

    def timed(fn, nbytes, name):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 100.0  # ms over 10 calls -> us per call
        out[name] = {"us_per_call": round(us, 2), "bytes": nbytes, "gbps": round(nbytes / us / 1e3, 1)}

    timed(lambda: torch.sum(x, dtype=torch.float32), 2 * n, "sum_bf16_4GiB")
    # the vendor BLAS matrix-vector product: a 4 GiB bf16 matrix read once
    mat = x.view(1 << 16, 1 << 15)
    vec = torch.ones(1 << 15, dtype=torch.bfloat16, device="cuda")
    timed(lambda: torch.mv(mat, vec), 2 * n, "gemv_bf16_4GiB")
    src = x[: 1 << 29]
    dst = torch.empty_like(src)
    timed(lambda: dst.copy_(src), 2 * 2 * (1 << 29), "copy_1GiB")
    print(json.dumps({"read_probe": out, "peak_gbps": HBM_PEAK_GBPS}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--slices", type=int, default=None,
                    help="attention split: -T = batch-invariant chunks of T 32-key tiles (the lossless R-ISD "
                         "configuration; default T = 64 for 8b, 66 for 32b); 0 = stream-K with automatic "
                         "slices; S > 0 = stream-K with S workgroups per KV-head group")
    ap.add_argument("--proposal", choices=("sample", "argmax"), default="sample",
                    help="draft proposals: sampled from q (default) or argmax q")
    ap.add_argument("--lora", choices=("gated", "off"), default="gated",
                    help="projections with the gated LoRA of R-ISD (default) or the base GEMM alone "
                         "(the ratio of the two step times is the LoRA overhead alpha)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (one per step, holding that step's logits "
                         f"rows); every {PROBE_EVERY}th timed step runs eagerly with the event probes")
    ap.add_argument("--workload", choices=("8b", "8b1", "32b"), default="8b",
                    help="8b: C=64 ragged 1k-8k contexts, 36 layers (default); 8b1: one sequence of 4,096 cached "
                         "tokens, 36 layers; 32b: C=16 contexts of 16,384, 64 layers of 64/8 heads, hidden 5120")
    ap.add_argument("--N", type=int, default=4, help="stride N (2N-row blocks); default 4")
    ap.add_argument("--accept", type=float, default=0.9, choices=(0.5, 0.7, 0.9),
                    help="mean per-draft acceptance the draft noise is set for; default 0.9")
    ap.add_argument("--kv", choices=("commit", "write"), default="commit",
                    help="commit (default): attention reads the block's own K/V from its rows and one "
                         "isd_kv_write_layers after the accept writes the accepted rows of every layer; write: "
                         "isd_kv_write of the whole block before each attention call")
    ap.add_argument("--no-lm-head", action="store_true",
                    help="skip the LM-head leg (isd_lm_head timed after the steps; not part of the step)")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the whole-forward leg (every layer with its MLP, LM head, accept on its statistics; "
                         "rank 32 and 128 against the base projections)")
    ap.add_argument("--forward-steps", type=int, default=6, help="timed steps of each whole-forward configuration")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for counter scaling)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only time vendor streaming kernels (a 4 GiB bf16 sum and matrix-vector product, a 1 GiB copy) on HIP events: "
                         "the read rate the chip gives a plain stream, beside the attention's")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-kernel means of a rocprofv3 --pmc CSV output directory and exit")
    ap.add_argument("--algo-out", metavar="FILE",
                    help="write the algorithmic bytes of every step's attention call and accept to FILE (JSON)")
    ap.add_argument("--traffic-report", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR", "ALGO_JSON"),
                    help="HBM traffic report from FETCH_SIZE / WRITE_SIZE counter runs of the step and of "
                         "--copy-probe, against the --algo-out bytes of the profiled run, and exit")
    args = ap.parse_args()
    if args.traffic_report:
        traffic_report(*args.traffic_report)
        return
    if args.slices is None:
        # The chunk size is a deployment constant picked for the context mix:
        # at 16,384-token contexts, 66 tiles give 8 chunks per sequence and
        # 16 x 8 x 2 head groups = 256 workgroups, one round on 256 CUs
        # (64 tiles would give a ninth, one-tile chunk and 288 workgroups);
        # one sequence of 4,096 tokens runs fastest with 8-tile chunks (17
        # chunks per KV head, one head per workgroup).
        args.slices = {"8b": -64, "8b1": -8, "32b": -66}[args.workload]
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.read_probe:
        read_probe()
        return
    if args.copy_probe:
        torch.cuda.set_device(0)
        n = 1 << 29  # 2-byte elements: 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 2 * n, "copy_probe_bytes_written": 2 * n, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no multi-GPU "
              "path; the step shards over sequences with no exchange, so N GPUs run N copies of it",
              file=sys.stderr)
        sys.exit(2)

    import draft_verify_decoding_amd as dvd

    cfg = dict({"8b": CFG, "8b1": CFG_8B1, "32b": CFG_32B}[args.workload], proposal=args.proposal, lora=args.lora,
               N=args.N, accept=args.accept)
    commit_mode = args.kv == "commit"
    default_workload = args.workload == "8b" and args.N == 4
    dev = "cuda"
    torch.cuda.set_device(0)
    dvd.lib()
    K, W = args.steps, args.warmup
    total = K + W
    C, N, Hq, D, L, V = cfg["C"], cfg["N"], cfg["Hq"], cfg["D"], cfg["layers"], cfg["V"]
    R = 2 * N

    t_setup = time.perf_counter()
    st = build(cfg, total, dev)
    log(f"[bench] inputs built in {time.perf_counter() - t_setup:.1f} s")
    logits, ctxs, nds, accs, final_ctx = dry_run(cfg, total, st["ctx0"], dev)
    log(f"[bench] trajectory fixed: {total} steps, mean accepted {accs.mean():.3f}")
    max_len = int(ctxs.max()) + R

    # prepared calls
    ctx = torch.from_numpy(st["ctx0"].astype(np.int32)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    att_ws = None
    need = dvd.isd_attention_workspace_size(st["kvs"][0], C, R, Hq, max_len, args.slices)
    if need:
        att_ws = torch.empty(need, dtype=torch.uint8, device=dev)
    layer_calls = []
    for l in range(L):
        lay, kv = st["layers"][l], st["kvs"][l]
        p = lay["proj"]
        lg = lambda name, x: (dvd.prepare_linear_gated(x, p[name]["W"], p[name]["A"], p[name]["B"], st["mask"],
                                                       p[name]["y"], st["lora_ws"]) if args.lora == "gated"
                              else dvd.prepare_linear(x, p[name]["W"], p[name]["y"]))
        layer_calls.append(dict(
            qkv=[lg("qkv", lay["x"])],
            kvw=None if commit_mode else dvd.prepare_kv_write(kv, lay["k"], lay["v"], ctx, dev_err=err),
            att=dvd.prepare_attention(kv, lay["q"], ctx, max_len, lay["out"], ws=att_ws, slices=args.slices,
                                      dev_err=err, k_blk=lay["k"] if commit_mode else None,
                                      v_blk=lay["v"] if commit_mode else None),
            o=lg("o", lay["xo"])))
    s_a, s_b = dvd.SeqState(C, N, dev), dvd.SeqState(C, N, dev)
    acc_ws = dvd.accept_workspace(C, N, V, R, device=dev)
    acc_out = dvd.AcceptOutputs(C, N, R, dev, diag=False)
    # commit mode: the contexts before the accept advances them are the
    # positions of the rows to commit, kv_commit their count
    ctx_prev = torch.empty_like(ctx)
    commit = (dvd.prepare_kv_write_layers(st["kvs"][0], st["layer_stride"], st["k_all"], st["v_all"], ctx_prev,
                                          acc_out.kv_commit, dev_err=err) if commit_mode else None)

    # every call runs on torch's current stream, so torch's events bracket
    # exactly the launches of that call. Events go on every PROBE_EVERY-th
    # timed step only: each recorded event costs GPU time between kernels,
    # which would otherwise inflate the step time the headline is based on.
    probes = list(range(0, K, PROBE_EVERY))
    ev = lambda: torch.cuda.Event(enable_timing=True)
    att_ev = [[(ev(), ev()) for _ in range(L)] for _ in probes]
    proj_ev = [[(ev(), ev(), ev()) for _ in range(L)] for _ in probes]
    acc_ev = [(ev(), ev()) for _ in probes]
    com_ev = [ev() for _ in probes]  # end of the KV commit (after the accept's end event)

    # --graph: the whole step on one side stream, captured once per step: each
    # step's graph holds that step's logits and the previous step's (the
    # pre-generated teacher rows stay where they are, so no copy runs), the
    # state buffers of its parity and its step number. Replayed in order.
    gs = torch.cuda.Stream() if args.graph else None
    if args.graph:
        with torch.cuda.stream(gs):
            layer_calls = []
            for l in range(L):
                lay, kv = st["layers"][l], st["kvs"][l]
                p = lay["proj"]
                lg = lambda name, x: (dvd.prepare_linear_gated(x, p[name]["W"], p[name]["A"], p[name]["B"],
                                                               st["mask"], p[name]["y"], st["lora_ws"])
                                      if args.lora == "gated" else dvd.prepare_linear(x, p[name]["W"], p[name]["y"]))
                layer_calls.append(dict(
                    qkv=[lg("qkv", lay["x"])],
                    kvw=None if commit_mode else dvd.prepare_kv_write(kv, lay["k"], lay["v"], ctx, dev_err=err),
                    att=dvd.prepare_attention(kv, lay["q"], ctx, max_len, lay["out"], ws=att_ws,
                                              slices=args.slices, dev_err=err, k_blk=lay["k"] if commit_mode else None,
                                              v_blk=lay["v"] if commit_mode else None),
                    o=lg("o", lay["xo"])))
            if commit_mode:
                commit = dvd.prepare_kv_write_layers(st["kvs"][0], st["layer_stride"], st["k_all"], st["v_all"],
                                                     ctx_prev, acc_out.kv_commit, dev_err=err)

    def step(t, timed_idx=None):
        if args.graph:
            with torch.cuda.stream(gs):
                if timed_idx is None:
                    graphs[t].replay()
                else:
                    body(t, timed_idx)
            return
        body(t, timed_idx)

    def body(t, timed_idx=None):
        for l in range(L):
            c = layer_calls[l]
            if timed_idx is not None:
                proj_ev[timed_idx][l][0].record()
            for f in c["qkv"]:
                f()
            if timed_idx is not None:
                proj_ev[timed_idx][l][1].record()
            if c["kvw"] is not None:
                c["kvw"]()
            if timed_idx is not None:
                att_ev[timed_idx][l][0].record()
            c["att"]()
            if timed_idx is not None:
                att_ev[timed_idx][l][1].record()
            c["o"]()
            if timed_idx is not None:
                proj_ev[timed_idx][l][2].record()
        s_in, s_out = (s_a, s_b) if t % 2 == 0 else (s_b, s_a)
        if commit is not None:
            ctx_prev.copy_(ctx)
        if timed_idx is not None:
            acc_ev[timed_idx][0].record()
        dvd.isd_accept(logits[t], logits[t - 1] if t else None, s_in, s_out, N, cfg["seed"], t, out=acc_out,
                       ws=acc_ws, ctx=ctx, dev_err=err, proposal=cfg["proposal"], stream=gs)
        if timed_idx is not None:
            acc_ev[timed_idx][1].record()
        if commit is not None:
            commit()
            if timed_idx is not None:
                com_ev[timed_idx].record()

    if args.graph:
        graphs = {}
        torch.cuda.synchronize()
        t_cap = time.perf_counter()
        for t in range(total):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                body(t)
            graphs[t] = g
        torch.cuda.synchronize()
        log(f"[bench] {total} steps captured as HIP graphs in {time.perf_counter() - t_cap:.1f} s")

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    ctx_start = ctx.cpu().numpy().copy()
    assert np.array_equal(ctx_start, ctxs[W]), "warmup diverged from the fixed trajectory"

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, timed_idx=i // PROBE_EVERY if i % PROBE_EVERY == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ctx_end = ctx.cpu().numpy()
    assert err.item() == 0, f"device error flags {err.item()}"
    assert np.array_equal(ctx_end, final_ctx), "timed run diverged from the fixed trajectory"
    tokens = int(np.sum(ctx_end - ctx_start))  # n_emit == kv_commit per sequence-step
    if args.algo_out:
        with open(args.algo_out, "w") as fh:
            json.dump({"attention_bytes_per_step": [attention_bytes(ctxs[t], cfg) for t in range(total)],
                       "accept_bytes_per_step": [accept_bytes(nds[t], accs[t], cfg) for t in range(total)],
                       "layers": L, "copy_probe_bytes": 2 * (1 << 29)}, fh)

    att_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in att_ev])  # [K, L]
    qkv_ms = np.array([[a.elapsed_time(b) for a, b, _ in row] for row in proj_ev])
    o_ms = np.array([[a_end.elapsed_time(c) for (_, _, c), (_, a_end) in zip(row, arow)]
                     for row, arow in zip(proj_ev, att_ev)])  # attention end -> O projection end
    acc_ms = np.array([a.elapsed_time(b) for a, b in acc_ev])
    com_ms = np.array([b.elapsed_time(c) for (a, b), c in zip(acc_ev, com_ev)]) if commit is not None else None
    att_bytes = np.array([attention_bytes(ctxs[W + i], cfg) for i in probes])  # per launch, per probed step
    acc_bytes = np.array([accept_bytes(nds[W + i], accs[W + i], cfg) for i in probes])
    att_gbps = float(np.sum(att_bytes * L) / np.sum(att_ms) / 1e6)
    acc_gbps = float(np.sum(acc_bytes) / np.sum(acc_ms) / 1e6)
    aa_gbps = float((np.sum(att_bytes * L) + np.sum(acc_bytes)) / (np.sum(att_ms) + np.sum(acc_ms)) / 1e6)
    ms_step = wall / K * 1e3
    value = tokens / wall
    probe_tokens = int(sum(np.sum(accs[W + i] + 1) for i in probes))  # n_emit = a + 1
    att_only_tps = probe_tokens / ((np.sum(att_ms) + np.sum(acc_ms)) / 1e3)

    res = {
        "metric": {"8b": METRIC,
                   "8b1": f"ISD accepted tokens/s at C=1,N={N} (8B shapes, context 4096); attn+accept HBM GB/s "
                          "vs peak",
                   "32b": f"ISD accepted tokens/s at C={C},N={N} (32B shapes); attn+accept HBM GB/s vs peak"}[
                       args.workload],
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"stationary batch C={C}, N={N} ({R}-row blocks), "
                         + ("32B-class GQA 64/8 heads, head_dim 128, 64 layers, hidden 5120, "
                            if args.workload == "32b" else
                            "8B-class GQA 32/8 heads, head_dim 128, 36 layers, hidden 4096, ")
                         + "bf16 paged KV (16-token pages), "
                         + {"8b": "contexts U{1024..8192}", "8b1": "context 4096",
                            "32b": "contexts 16384"}[args.workload]
                         + f", vocab 151936, acceptance ~{cfg['accept']}, "
                         + ("gated-LoRA rank-32" if args.lora == "gated" else "base (no LoRA)")
                         + " Q/K/V/O projections; MLP and LM head not included"),
            "C": C, "N": N, "layers": L, "Hq": Hq, "Hkv": cfg["Hkv"], "head_dim": D, "vocab": V,
            "global_batch": C, "seq_len": int(np.mean(ctxs[W])), "parallelism": "none (1 GPU)",
            "proposal": cfg["proposal"],
            "attention_split": ("batch-invariant, chunks of %d tiles" % -args.slices if args.slices < 0
                                else "stream-K, %s slices" % (args.slices or "automatic")),
            "projections": ("gated LoRA rank %d on MASK rows" % cfg["lora_rank"] if args.lora == "gated"
                            else "base GEMM only (no LoRA)"),
            "kv": ("block K/V read from its rows by the attention; accepted rows of all layers written after the "
                   "accept in one isd_kv_write_layers launch" if commit_mode
                   else "isd_kv_write of the whole block before each attention call"),
            "launch": ("HIP graph replay per step (every %dth timed step eager, with the event probes)" % PROBE_EVERY
                       if args.graph else "eager"),
        },
        "roofline": {
            "kernel": ("isd_attention_with_block" if commit_mode else "isd_attention")
                      + " (main + LSE merge launches of one call)",
            "bound": "hbm",
            "achieved": round(att_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
        "timing_probes": f"HIP events on {len(probes)} of the {K} timed steps (every {PROBE_EVERY}th)",
        "attention_ms_per_launch": round(float(att_ms.mean()), 5),
        "accept_ms_per_step": round(float(acc_ms.mean()), 5),
        "kv_commit_ms_per_step": round(float(com_ms.mean()), 5) if com_ms is not None else None,
        "accept_gbps": round(acc_gbps, 1),
        "accept_frac_of_peak": round(acc_gbps / HBM_PEAK_GBPS, 4),
        "attn_accept_gbps": round(aa_gbps, 1),
        "attn_accept_frac_of_peak": round(aa_gbps / HBM_PEAK_GBPS, 4),
        "attn_accept_only_tokens_per_s": round(float(att_only_tps), 1),
        "tokens_per_forward": round(tokens / (K * C), 4),
        "mean_accepted": round(float(accs[W:].mean()), 4),
    }
    qkv_flops, o_flops = projection_flops(cfg)
    res["projection_us_per_launch"] = {"qkv": round(float(qkv_ms.mean()) * 1e3, 2),
                                       "o": round(float(o_ms.mean()) * 1e3, 2)}
    proj_tflops = (qkv_flops + o_flops) * len(probes) * L / ((np.sum(qkv_ms) + np.sum(o_ms)) / 1e3) / 1e12
    res["projection_mfma"] = {"achieved": round(float(proj_tflops), 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(float(proj_tflops) / MFMA_BF16_PEAK_TFLOPS, 4)}
    rec = committed_traffic() if default_workload else None
    if rec is not None:
        # counter bytes per call of the profiled run, and their ratio to that
        # run's algorithmic bytes (contexts grow a little over a run)
        res["roofline"]["traffic"] = rec["hbm_bytes_per_call"]
        res["roofline"]["traffic_over_algorithmic"] = rec["ratio_to_algorithmic"]
        res["roofline"]["traffic_source"] = os.path.relpath(TRAFFIC_FILE, ROOT)
    if not args.no_lm_head:
        del logits[:]
        torch.cuda.empty_cache()
        res["lm_head"] = lm_head_leg(cfg, dev)
    if not args.no_forward and args.workload in ("8b", "8b1"):
        del logits[:]
        torch.cuda.empty_cache()
        res["forward"] = forward_leg(cfg, st, dev, args.slices, steps=args.forward_steps)
    if not args.no_cpu_baseline:
        t_cpu = time.perf_counter()
        res["cpu_baseline"] = {"8b": lambda: cpu_baseline(cfg),
                               "8b1": lambda: cpu_baseline(cfg, fwd_seqs=8, accept_seqs=48, accept_steps=14),
                               "32b": lambda: cpu_baseline(cfg, fwd_seqs=1, accept_seqs=16, accept_steps=14,
                                                           layers_timed=8)}[args.workload]()
        log(f"[bench] cpu baseline took {time.perf_counter() - t_cpu:.1f} s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

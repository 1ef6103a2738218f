"""The forward around the ISD step: RMSNorm, the SwiGLU MLP, bf16 rounding
and one decoder block composed from the other oracle modules (oracle side).

Test infrastructure, plain numpy in float64 (bf16 rounding through torch's
CPU conversion, a library routine); it shares no code with the HIP path.

What the pages fix: the released I-DLM models are built on Qwen3-8B and
Qwen3-32B ("Documentation et ressources > Model Zoo" on the I-DLM page,
fr.news.hada.io), converted from AR models with causal attention and a
logit shift ("Méthodologie d'I-DLM"), so one ISD step is one causal
forward of such a model over the stride block. The pages do not describe
the block itself. Readings, the plainest ones for that model family:
  * pre-norm decoder block: h += O(attn(QKV(norm(h)))), then
    h += Down(silu(Gate(norm(h))) * Up(norm(h))); a final norm before the
    LM head;
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, eps = 1e-6;
  * silu(z) = z / (1 + exp(-z));
  * the gated LoRA of lossless R-ISD on the Q, K, V and O projections
    only ("Lossless R-ISD");
  * no positional encoding inside the block (the attention oracle takes
    q and k as they enter the attention, i.e. after any rotary encoding);
  * activations cross kernel boundaries in bf16, the residual stream stays
    in fp32: the values are rounded to bf16 where the forward hands them to
    a bf16 operand (the normalised rows, q / k / v, the attention output,
    the MLP activation, the logits).
"""

import numpy as np
import torch

from . import accept, attention, lora

EPS = 1e-6


def bf16_round(x):
    """Round to bfloat16 (nearest, ties to even) through fp32, back to fp64."""
    t = torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def rmsnorm(x, g, eps=EPS):
    """x / sqrt(mean over the last axis of x^2 + eps) * g."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gate, up):
    """silu(gate) * up, elementwise."""
    return silu(gate) * np.asarray(up, np.float64)


def block(h, p, kv, ctx, is_mask, N, lora_scale=1.0):
    """One decoder block on the rows of a stride-block batch.

    h        float64 [C*R, H] residual stream (R = 2N rows per sequence)
    p        dict of float64 weights: g1, g2 [H]; Wqkv [(Hq+2Hkv)D, H];
             Aqkv, Bqkv (gated LoRA of Q|K|V); Wo [H, Hq D]; Ao, Bo;
             Wgu [2I, H] (gate rows then up rows); Wd [H, I]; and the
             head counts Hq, Hkv, D
    kv       (k_pages, v_pages, table) float64 pages [P, 16, Hkv, D] that
             hold each sequence's cached positions 0 .. ctx-1
    ctx      [C] cached tokens before the block
    Returns (h_out, intermediates dict).
    """
    Hq, Hkv, D = p["Hq"], p["Hkv"], p["D"]
    M = h.shape[0]
    R = 2 * N
    C = M // R
    x = bf16_round(rmsnorm(h, p["g1"]))
    qkv = lora.gated_lora(x, p["Wqkv"], p["Aqkv"], p["Bqkv"], is_mask, lora_scale)
    q = bf16_round(qkv[:, : Hq * D]).reshape(C, R, Hq, D)
    k = bf16_round(qkv[:, Hq * D:(Hq + Hkv) * D]).reshape(C, R, Hkv, D)
    v = bf16_round(qkv[:, (Hq + Hkv) * D:]).reshape(C, R, Hkv, D)
    # the block's own K/V join the cached ones at positions ctx .. ctx+R-1
    kp, vp, table = (a.copy() for a in kv)
    attention.kv_write(kp, vp, table, ctx, k, v, np.full(C, R))
    o = attention.block_attention(q, kp, vp, table, ctx)
    ob = bf16_round(o.reshape(M, Hq * D))
    h1 = h + lora.gated_lora(ob, p["Wo"], p["Ao"], p["Bo"], is_mask, lora_scale)
    x2 = bf16_round(rmsnorm(h1, p["g2"]))
    gu = lora.linear(x2, p["Wgu"])
    I = gu.shape[1] // 2
    act = bf16_round(swiglu(gu[:, :I], gu[:, I:]))
    d = lora.linear(act, p["Wd"])
    h2 = h1 + d
    return h2, dict(x=x, qkv=qkv, q=q, k=k, v=v, o=o, ob=ob, h1=h1, x2=x2, gu=gu, act=act, d=d)


def lm_head(h, g, W, chunk=8192):
    """Final norm, then logits = bf16(norm(h) W^T) and their per-chunk
    softmax statistics (accept.chunk_stats of every row)."""
    xf = bf16_round(rmsnorm(h, g))
    logits = bf16_round(lora.linear(xf, W))
    stats = np.stack([accept.chunk_stats(row, chunk) for row in logits])
    return xf, logits, stats

"""A whole synthetic forward of the ISD step through the library: for every
decoder layer, RMSNorm -> gated Q|K|V projection -> bf16 q, k, v -> causal
attention of the block over the paged cache (bf16 out) -> gated O projection ->
residual add and RMSNorm -> gate|up projection -> SwiGLU -> down projection;
then the final RMSNorm and the LM head, whose chunk statistics feed the
accept step. Every step is a library call (argument marshalling only); the
calls are prepared once and replayed.

The block structure is the usual pre-norm one of the base model family the
pages name (Qwen3-8B / 32B, I-DLM page, "Documentation et ressources >
Model Zoo"); the pages do not describe it.
"""

import torch

from . import (KVCache, accept_workspace, isd_attention_workspace_size, isd_lm_head_workspace_size,
               isd_lora_workspace_size, lora_workspace, prepare_attention, prepare_cast_bf16, prepare_linear, prepare_linear_gated,
               prepare_lm_head, prepare_rmsnorm, prepare_swiglu)


class LayerWeights:
    """bf16 weights of one decoder layer (Q|K|V fused, gate|up fused).

    The gated LoRA of Q, K and V is either one stacked adapter on the fused
    projection (Aqkv [3r, H], Bqkv block-diagonal [(Hq+2Hkv)D, 3r]) or, when
    `qkv_adapters` is given as three (A, B) pairs, one adapter per
    projection; Q, K and V then run as three projections (the adapter's rank
    is at most 128 per call)."""

    def __init__(self, g1, g2, Wqkv, Wo, Wgu, Wd, Aqkv=None, Bqkv=None, Ao=None, Bo=None, qkv_adapters=None):
        self.g1, self.g2, self.Wqkv, self.Wo, self.Wgu, self.Wd = g1, g2, Wqkv, Wo, Wgu, Wd
        self.Aqkv, self.Bqkv, self.Ao, self.Bo = Aqkv, Bqkv, Ao, Bo
        self.qkv_adapters = qkv_adapters


class Forward:
    """Prepared calls of one forward over C sequences of R = 2N block rows.

    layers   list of LayerWeights
    kvs      one KVCache per layer (pages hold each sequence's cached
             positions below ctx)
    ctx      int32 [C] device tensor (read at call time)
    mask     uint8 [C*R] MASK rows (the gated LoRA's rows)
    gf, Wlm  final norm gain [H] and LM head [V, H] (bf16)
    k_all, v_all  bf16 [L, C, R, Hkv, D]: the block's K/V rows of every
             layer, kept for the KV commit after the accept
    lora     "gated" (R-ISD adapters on Q|K|V and O) or "off"
    """

    def __init__(self, layers, kvs, ctx, mask, gf, Wlm, C, N, Hq, Hkv, D, max_len, slices, k_all, v_all,
                 lora="gated", dev_err=None, dev="cuda"):
        R = 2 * N
        M = C * R
        H = layers[0].Wqkv.shape[1]
        I = layers[0].Wd.shape[1]
        V = Wlm.shape[0]
        f32, bf = torch.float32, torch.bfloat16
        e = lambda *s, dt=f32: torch.empty(s, dtype=dt, device=dev)
        self.h = e(M, H)
        self.x, self.x2, self.xf = e(M, H, dt=bf), e(M, H, dt=bf), e(M, H, dt=bf)
        nq = (Hq + 2 * Hkv) * D
        self.yqkv, self.q = e(M, nq), e(C, R, Hq, D, dt=bf)
        # attention writes its bf16 output straight into the O projection's input
        self.ob, self.yo = e(M, Hq * D, dt=bf), e(M, H)
        self.gu, self.act, self.yd = e(M, 2 * I), e(M, I, dt=bf), e(M, H)
        # two logits buffers, alternated step by step: the accept step reads
        # the previous step's block for its residual draws
        self.logits_buf = [e(C, R, V, dt=bf), e(C, R, V, dt=bf)]
        self.logits = self.logits_buf[0]
        self.nch = (V + 8191) // 8192
        self.stats = e(C, R, self.nch, 2)
        ranks = [w.Ao.shape[0] for w in layers if w.Ao is not None]
        ranks += [w.Aqkv.shape[0] for w in layers if w.Aqkv is not None]
        ranks += [a.shape[0] for w in layers if w.qkv_adapters for a, _ in w.qkv_adapters]
        r_max = max([0] + ranks)
        split = layers[0].qkv_adapters is not None
        widths = [Hq * D, Hkv * D, Hkv * D]
        self.lora_ws = lora_workspace(M, max(r_max, 16), dev)  # zero-filled
        need = isd_attention_workspace_size(kvs[0], C, R, Hq, max_len, slices)
        self.att_ws = e(max(need, 256) // 4 + 1)
        self.lm_ws = e(isd_lm_head_workspace_size(M, V) // 4 + 1)
        self.calls = []
        prev_delta = None
        for l, w in enumerate(layers):
            c = self.calls
            c.append(prepare_rmsnorm(self.h, w.g1, self.x, delta=prev_delta))
            if split:  # each projection rounds its own output to bf16 q, k or v
                r0 = 0
                dsts = (self.q, k_all[l], v_all[l])
                for j, (wd, dst) in enumerate(zip(widths, dsts)):
                    Wj, yj = w.Wqkv[r0:r0 + wd], dst.view(M, wd)
                    if lora == "gated":
                        A, B = w.qkv_adapters[j]
                        c.append(prepare_linear_gated(self.x, Wj, A, B, mask, yj, self.lora_ws))
                    else:
                        c.append(prepare_linear(self.x, Wj, yj))
                    r0 += wd
            else:
                if lora == "gated":
                    c.append(prepare_linear_gated(self.x, w.Wqkv, w.Aqkv, w.Bqkv, mask, self.yqkv, self.lora_ws))
                else:
                    c.append(prepare_linear(self.x, w.Wqkv, self.yqkv))
                c.append(prepare_cast_bf16(self.yqkv, [self.q, k_all[l], v_all[l]]))
            c.append(prepare_attention(kvs[l], self.q, ctx, max_len, self.ob.view(C, R, Hq, D), ws=self.att_ws,
                                       slices=slices, dev_err=dev_err, k_blk=k_all[l], v_blk=v_all[l]))
            if lora == "gated":
                c.append(prepare_linear_gated(self.ob, w.Wo, w.Ao, w.Bo, mask, self.yo, self.lora_ws))
            else:
                c.append(prepare_linear(self.ob, w.Wo, self.yo))
            c.append(prepare_rmsnorm(self.h, w.g2, self.x2, delta=self.yo))
            c.append(prepare_linear(self.x2, w.Wgu, self.gu))
            c.append(prepare_swiglu(self.gu, self.act))
            c.append(prepare_linear(self.act, w.Wd, self.yd))
            prev_delta = self.yd
        self.calls.append(prepare_rmsnorm(self.h, gf, self.xf, delta=prev_delta))
        self.lm_head_calls = [prepare_lm_head(self.xf, Wlm, lg.view(M, V), self.stats.view(M, self.nch, 2),
                                              self.lm_ws) for lg in self.logits_buf]

    def __call__(self, h0, parity=0):
        """Runs the forward from the residual stream h0 [C*R, H] (fp32, the
        block's embeddings); leaves the logits in self.logits_buf[parity]
        (also self.logits) and their chunk statistics in self.stats."""
        self.h.copy_(h0)
        for f in self.calls:
            f()
        self.lm_head_calls[parity]()
        self.logits = self.logits_buf[parity]

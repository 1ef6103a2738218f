"""Paged KV cache write and causal GQA attention of the stride block (oracle).

Test infrastructure, plain numpy in float64; it shares no code with the HIP
path. What the pages fix, and where:

* The attention is strictly causal, which is what lets the model run in an
  AR serving stack (I-DLM, fr.news.hada.io, "Méthodologie d'I-DLM > Serving
  compatible AR"; the Hacker News thread on the same page adds that the
  structure stays causal with no denoising loop).
* The serving stack keeps K/V in a paged cache and uses an attention kernel
  that reads only from pages (same page, "Documentation et ressources >
  Serving (SGLang)"), so the block's own K/V are written to pages first.

Readings where the pages are silent: scale 1/sqrt(D); no positional
encoding, bias or window inside the operation; grouped-query heads map query
head h to KV head h // (Hq // Hkv); block row i of a sequence with ctx cached
tokens sits at position ctx + i and sees positions 0..ctx + i.

Layout used here (the plain one, not the kernel's): pages are
[num_pages, page_size, Hkv, D]; block_table[b, p] is the physical page that
holds positions p*page_size .. p*page_size + page_size - 1 of sequence b.
"""

import numpy as np


def kv_write(k_pages, v_pages, block_table, pos0, k_rows, v_rows, nrows):
    """Write rows r < nrows[b] of k_rows/v_rows [C, rows, Hkv, D] at positions
    pos0[b] + r of sequence b. Pages are updated in place."""
    ps = k_pages.shape[1]
    C = k_rows.shape[0]
    for b in range(C):
        for r in range(int(nrows[b])):
            pos = int(pos0[b]) + r
            page = int(block_table[b, pos // ps])
            k_pages[page, pos % ps] = k_rows[b, r]
            v_pages[page, pos % ps] = v_rows[b, r]


def gather_sequence(pages, block_table_row, length):
    """Logical [length, Hkv, D] view of one sequence, gathered page by page."""
    ps = pages.shape[1]
    pos = np.arange(length)
    return pages[block_table_row[pos // ps], pos % ps]


def block_attention(q, k_pages, v_pages, block_table, ctx, scale=None):
    """O[b, i, h] = sum_{t <= ctx_b + i} softmax_t(q . k_t * scale) v_t.

    q [C, R, Hq, D]; returns float64 [C, R, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    C, R, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((C, R, Hq, D), dtype=np.float64)
    for b in range(C):
        L = int(ctx[b]) + R
        K = gather_sequence(k_pages, block_table[b], L).astype(np.float64)
        V = gather_sequence(v_pages, block_table[b], L).astype(np.float64)
        visible = np.arange(L)[None, :] <= (int(ctx[b]) + np.arange(R))[:, None]
        for h in range(Hq):
            g = h // group
            s = (q[b, :, h, :] @ K[:, g, :].T) * scale  # [R, L]
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ V[:, g, :]
    return out

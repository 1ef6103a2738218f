/*
 * isd.h - C ABI of the Introspective Strided Decoding (ISD) step on MI355X.
 *
 * One ISD step of an I-DLM model runs a single causal forward over a stride
 * block of 2N rows: it verifies the N-1 drafts proposed on the previous step
 * with the min(1, p(x)/q(x)) test and proposes new tokens at MASK positions
 * (I-DLM - Modeles de langage a diffusion introspective, fr.news.hada.io,
 * sections "Methodologie d'I-DLM > Introspective Strided Decoding (ISD)" and
 * "Documentation et ressources > Inference & ISD"). This library implements
 * the data-parallel hot path of that step for one GPU (gfx950):
 *
 *   isd_kv_write      put the block's K/V rows into the paged cache
 *   isd_attention     causal GQA attention of the block over the pages
 *   isd_attention_with_block  the same, the block's own K/V taken from its rows
 *   isd_kv_write_layers  isd_kv_write for every layer of a model in one launch
 *   isd_accept        vocab softmax, p/q test, residual / bonus draw, proposals
 *   isd_block_assemble  the next step's block: newest token, drafts, MASK
 *   isd_linear        y = x W^T (bf16 in, fp32 or bf16 out), the base projection
 *   gated_lora_apply  y += s (x A^T) B^T on MASK rows only (R-ISD)
 *   isd_linear_gated  both of the above in one pass
 *   isd_lm_head       logits = h W^T (bf16) with their softmax chunk statistics
 *   isd_rmsnorm, isd_cast_bf16, isd_swiglu
 *                     the normalisation, cast and activation steps of the
 *                     decoder block around them
 *
 * Conventions shared by every call:
 *   - Every pointer argument is device memory owned by the caller, except
 *     the struct pointers themselves (host memory, read during the call).
 *     The library never allocates device memory; calls that need scratch
 *     space take a caller-provided workspace and publish its size.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     never synchronises. Calls are stateless and thread-safe; two calls that
 *     share a workspace must not overlap.
 *   - Return value: ISD_OK, or a negative ISD_E_* code when an argument is
 *     invalid or unsupported (checked on the host before any launch) or a
 *     launch fails. isd_strerror() gives the text.
 *   - Problems only the device can see (a page id outside the pool, a
 *     position beyond a sequence's block table, a non-finite logits row, a
 *     draft id outside the vocabulary, an invalid per-sequence state) are
 *     ORed as ISD_DEV_* bits into *dev_err when dev_err is not NULL; kernels
 *     never trap. The caller clears dev_err.
 *   - Element types: ISD_BF16 (bfloat16 bits in uint16) or ISD_F32.
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ codes */
#define ISD_OK 0
#define ISD_E_INVALID (-1)     /* null pointer, size or stride out of range */
#define ISD_E_UNSUPPORTED (-2) /* dtype, head_dim, stride, rank or shape not built */
#define ISD_E_WORKSPACE (-3)   /* workspace missing or too small */
#define ISD_E_LAUNCH (-4)      /* the HIP runtime refused a launch */
#define ISD_E_DEVICE (-5)      /* the current device is not a gfx950 GPU */

#define ISD_DEV_PAGE_OOB 1u    /* block-table entry outside [0, num_pages) */
#define ISD_DEV_CAPACITY 2u    /* position beyond the block table's columns */
#define ISD_DEV_NONFINITE 4u   /* a logits row read by isd_accept holds NaN/Inf */
#define ISD_DEV_TOKEN_OOB 8u   /* a pending draft id outside [0, V) */
#define ISD_DEV_STATE 16u      /* n_draft or q_row out of range */

#define ISD_BF16 1
#define ISD_F32 2

/* Proposal rule of isd_accept (see there). */
#define ISD_PROPOSE_SAMPLE 0 /* drafts drawn from q, verified with min(1, p/q) */
#define ISD_PROPOSE_ARGMAX 1 /* drafts = argmax q (a point mass)            */

#define ISD_PAGE_SIZE 16 /* tokens per KV page */

const char* isd_strerror(int code);
/* Library version as 10000*major + 100*minor + patch. */
int isd_version(void);

/* --------------------------------------------------------- KV cache
 * Paged KV cache (I-DLM page, "Documentation et ressources > Serving
 * (SGLang)": paged KV and an attention kernel that reads only from pages).
 *
 * Physical layout of one page, chosen so that every MFMA operand the
 * attention kernel needs is a run of 16 contiguous bytes:
 *   K: [num_kv_heads][head_dim / KP][16 slots][KP]    KP = 16 / sizeof(elem)
 *   V: [num_kv_heads][2 half-pages][head_dim][8 slots]
 * i.e. for bf16, element (slot s, head g, dim d) of page p is at
 *   k_pages[((p*Hkv + g)*(D/8) + d/8)*16*8 + s*8 + d%8]
 *   v_pages[((p*Hkv + g)*2 + s/8)*D*8 + d*8 + s%8].
 * Position t of sequence b lives in page block_table[b*table_stride + t/16],
 * slot t%16. Entries of the block table past a sequence's length are never
 * read.
 */
typedef struct isd_kv_cache {
  void* k_pages;              /* num_pages * Hkv * D * 16 elements */
  void* v_pages;              /* num_pages * Hkv * D * 16 elements */
  const int32_t* block_table; /* [C][table_stride] physical page ids */
  int32_t table_stride;       /* columns of block_table (max pages per sequence) */
  int32_t num_pages;          /* pages in each pool */
  int32_t page_size;          /* must be ISD_PAGE_SIZE */
  int32_t num_kv_heads;       /* Hkv, 1..64 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t dtype;              /* ISD_BF16 or ISD_F32 */
} isd_kv_cache;

/* Write K/V rows into the pages: row r < nrows[b] of sequence b goes to
 * position pos0[b] + r. k and v are [C][rows][Hkv][D] in kv->dtype.
 * nrows may be NULL (every sequence writes `rows` rows). Positions whose
 * page column is >= table_stride or whose page id is outside the pool are
 * skipped and flagged (ISD_DEV_CAPACITY / ISD_DEV_PAGE_OOB); a negative
 * position is skipped and flagged ISD_DEV_STATE. Every other slot of the
 * pages keeps its value. Two sequences of one call must not write into the
 * same page (a page's V slots are rewritten in runs of 8). C <= 65535
 * (else ISD_E_UNSUPPORTED); k and v must be 16-byte aligned. */
int isd_kv_write(const isd_kv_cache* kv, const void* k, const void* v,
                 const int32_t* pos0, const int32_t* nrows, int C, int rows,
                 int32_t* dev_err, hipStream_t stream);

/* isd_kv_write_layers: isd_kv_write for `layers` layers that share the
 * block table and the pool geometry of `kv` (layer 0): layer l's pools start
 * l * layer_stride elements after kv->k_pages / kv->v_pages (layer_stride >=
 * the elements of one pool when layers > 1), and its rows l * C * rows * Hkv
 * * D elements after k / v ([layers][C][rows][Hkv][D]). pos0 and nrows are
 * shared by all layers. This is the KV commit of a step: after isd_accept,
 * nrows = kv_commit and pos0 = the contexts before the commit write exactly
 * the accepted rows of every layer. Errors: as isd_kv_write, and
 * ISD_E_INVALID for a negative count or overlapping pools,
 * ISD_E_UNSUPPORTED for more than 65535 layers.
 */
int isd_kv_write_layers(const isd_kv_cache* kv, int layers,
                        int64_t layer_stride, const void* k, const void* v,
                        const int32_t* pos0, const int32_t* nrows, int C,
                        int rows, int32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------- attention
 * Causal grouped-query attention of the stride block over the paged cache
 * (strict causality: I-DLM page, "Methodologie d'I-DLM > Serving compatible
 * AR"). Row i of sequence b sits at position ctx[b] + i and attends to
 * positions 0 .. ctx[b] + i, all read from pages: the block's own K/V must
 * have been written with isd_kv_write first.
 *
 *   q    [C][rows][Hq][D] in kv->dtype
 *   out  [C][rows][Hq][D] normalised attention output: fp32 (odtype
 *        ISD_F32) or the fp32 value rounded to bf16, nearest even
 *        (ISD_BF16); 16-byte aligned. Partial results stay fp32.
 *   ctx  [C] cached tokens before the block
 *   Query head h reads KV head h / (Hq / Hkv). scale multiplies q.k
 *   (1/sqrt(D) in the usual model). max_len is a host-side upper bound of
 *   ctx[b] + rows, used to size the launch and the workspace. The 32-key
 *   tiles of all sequences are split evenly over `slices` workgroups per
 *   group of KV heads (0 = automatic: 1536 waves over the chip, i.e. a
 *   workgroup on three CUs in four for 8B and 32B shapes);
 *   sequences shared by several workgroups are merged with a log-sum-exp
 *   combine in a fixed order, so results do not depend on scheduling (but
 *   do depend on the rest of the batch, through the split).
 *   slices = ISD_ATTN_INVARIANT(t), 1 <= t <= 65536, selects the
 *   batch-invariant split instead: every sequence is cut into chunks of t
 *   tiles (32t keys) from position 0, one workgroup per chunk (it runs
 *   best while a call's chunks do not outnumber the CUs), merged in chunk
 *   order. Then row i of sequence b is bit for bit equal to the same query
 *   sent as a one-row call with ctx[b] + i cached tokens and the same t, in
 *   any batch: the
 *   reduction order of the clean rows of a stride block is that of the
 *   autoregressive forward, which the bit-identical output of lossless
 *   R-ISD needs (I-DLM page, "Speedup Factor Explorer" and "Documentation
 *   et ressources > Lossless R-ISD"). In this mode ctx[b] + rows must not
 *   exceed max_len: a sequence that does is left unwritten and flags
 *   ISD_DEV_CAPACITY.
 *   The workspace (size from isd_attention_workspace_size with the same
 *   arguments) holds the partial results; no initialisation.
 * Supported: D in {64, 128}; Hq multiple of Hkv; (Hq/Hkv)*rows <= 128;
 * rows <= 64; C <= 8192; in the batch-invariant split also
 * C * ceil(ceil(max_len / 32) / t) * Hkv <= INT_MAX (else
 * ISD_E_UNSUPPORTED).
 */
#define ISD_ATTN_INVARIANT(chunk_tiles) (-(chunk_tiles))
size_t isd_attention_workspace_size(int C, int rows, int num_q_heads,
                                    const isd_kv_cache* kv, int max_len,
                                    int slices);
int isd_attention(const isd_kv_cache* kv, const void* q, const int32_t* ctx,
                  int C, int rows, int num_q_heads, float scale, int max_len,
                  int slices, void* out, int odtype, void* ws,
                  size_t ws_bytes, int32_t* dev_err, hipStream_t stream);

/* isd_attention_with_block: isd_attention where keys ctx[b] .. ctx[b] +
 * rows - 1, the block's own rows, are read from k and v ([C][rows][Hkv][D]
 * in kv->dtype, 16-byte aligned) instead of the pages, so the pages need to
 * hold only positions below ctx[b] (and the block table to cover them). The
 * output equals, bit for bit, isd_kv_write of k and v at ctx followed by
 * isd_attention; the pages are only read. A step can then attend first and
 * commit afterwards only the accepted rows (isd_kv_write_layers), with no
 * write into the pools between the layers' attention calls. Same
 * arguments, workspace and limits as isd_attention otherwise; ISD_E_INVALID
 * for a null or misaligned k, v.
 */
int isd_attention_with_block(const isd_kv_cache* kv, const void* k,
                             const void* v, const void* q, const int32_t* ctx,
                             int C, int rows, int num_q_heads, float scale,
                             int max_len, int slices, void* out, int odtype,
                             void* ws, size_t ws_bytes, int32_t* dev_err,
                             hipStream_t stream);

/* ---------------------------------------------------------- accept
 * Per-sequence decoding state carried from step to step. Draft j (1-based)
 * was proposed from row q_row + j - 1 of the previous step's block; q_x is
 * its probability under that row and (q_m, q_s) are that row's max logit
 * and sum of exp(l - q_m).
 */
typedef struct isd_seq_state {
  int32_t* n_draft; /* [C] pending drafts: 0 (FRESH) .. N-1 (FULL) */
  int32_t* drafts;  /* [C][N-1] draft token ids */
  float* q_x;       /* [C][N-1] Q_j(x_j) */
  float* q_m;       /* [C][N-1] */
  float* q_s;       /* [C][N-1] */
  int32_t* q_row;   /* [C] */
} isd_seq_state;

/* The accept side of one step (I-DLM page, "Documentation et ressources >
 * Inference & ISD": proposals q at MASK positions, verification p at clean
 * positions, keep x with probability min(1, p(x)/q(x))). For each sequence
 * with n = n_draft pending drafts, rows 0..n of the block are clean and rows
 * n+1.. are MASK rows (logit shift: row i predicts position ctx + i + 1):
 *   1. P_j = softmax(logits row j) in fp32 from the bf16/f32 logits.
 *   2. for j = 1..n: accept x_j iff u_j * q_x_j < P_{j-1}(x_j); a = number
 *      accepted before the first rejection.
 *   3. a < n: draw t from normalize(max(0, P_a - Q_{a+1})) (P_a if that mass
 *      is 0), next state FRESH (n_draft = 0).
 *      a = n: draw the bonus t from P_n and N-1 new drafts from rows
 *      n+1..n+N-1, next state FULL (n_draft = N-1, q_row = n+1).
 *   4. emit = (x_1..x_a, t), n_emit = kv_commit = a + 1.
 * With proposal = ISD_PROPOSE_ARGMAX (the argmax proposal of the pages'
 * serving stack, "Documentation et ressources > Serving (SGLang)") the new
 * drafts are argmax of rows n+1..n+N-1 (ties to the smallest id) with
 * q_x = 1, so step 2 reads u_j < P_{j-1}(x_j) and the residual of step 3 is
 * P_a with x_{a+1} removed; prev_logits is then not read (may be NULL).
 * Draws are inverse-CDF over ascending token ids with u from Philox4x64-10:
 * key (seed, 0), counter (slot, b, step, 0), u = ((w0>>41) + 0.5) * 2^-23;
 * slots 1..N-1 test drafts, slot N draws t, slot N+k draws proposal k.
 * A sequence whose step cannot be taken (non-finite row, bad draft id or
 * state) gets accepted = -1, n_emit = kv_commit = 0, emit = -1 and its state
 * copied unchanged, and a bit in dev_err.
 */
typedef struct isd_accept_args {
  int32_t C;     /* sequences, <= 65535 */
  int32_t N;     /* stride, 2..8 */
  int32_t V;     /* vocabulary size, <= 524288 */
  int32_t rows;  /* rows per block in logits (>= 2N-1, usually 2N) */
  int32_t dtype; /* logits element type */
  const void* logits;      /* [C][rows][ld] this step's block */
  const void* prev_logits; /* [C][rows][ld] previous block; NULL if no drafts */
  int64_t ld;              /* elements between rows, >= V, 16-byte aligned */
  isd_seq_state in;        /* read only */
  isd_seq_state out;       /* written; must not alias `in` */
  uint64_t seed;
  uint64_t step;
  int32_t* accepted;  /* [C] a, or -1 */
  int32_t* n_emit;    /* [C] */
  int32_t* emit;      /* [C][N], -1 past n_emit */
  int32_t* kv_commit; /* [C] */
  int32_t* ctx;       /* optional [C]: ctx[b] += kv_commit[b] (the commit) */
  float* p_x;         /* optional [C][N-1]: P_{j-1}(x_j) of tested drafts */
  float* resid_mass;  /* optional [C]: sum max(0, P_a - Q_{a+1}), or -1 */
  float* row_m;       /* optional [C][rows]: max logit of each row read */
  float* row_s;       /* optional [C][rows]: sum exp(l - row_m) */
  void* ws;           /* isd_accept_workspace_size(C, N, V, rows) bytes, 16-byte
                         aligned, caller-owned, contents on entry ignored */
  size_t ws_bytes;
  int32_t* dev_err;
  int32_t proposal;   /* ISD_PROPOSE_SAMPLE or ISD_PROPOSE_ARGMAX; the same on
                         consecutive steps of a sequence */
  const uint64_t* step_dev; /* optional: when not NULL the step number is read
                         from this device word and `step` is ignored, so one
                         captured HIP graph can be replayed step after step
                         (the caller advances the word between replays) */
  const float* chunk_stats; /* optional [C][rows][ceil(V/8192)][2]: the chunk
                         statistics of `logits` as isd_lm_head writes them;
                         when not NULL the statistics pass is skipped */
} isd_accept_args;

size_t isd_accept_workspace_size(int C, int N, int V, int rows);
int isd_accept(const isd_accept_args* args, hipStream_t stream);

/* isd_accept_noalloc: isd_accept for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). args->ws and args->ws_bytes are ignored: the workspace
 * is a fixed array in the library's device memory, one per GPU, of
 * isd_accept_noalloc_max_workspace() bytes (4 MiB), kept until the process
 * ends. The call allocates nothing. A call whose
 * isd_accept_workspace_size(C, N, V, rows) exceeds that maximum returns
 * ISD_E_WORKSPACE without launching. Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller. Results are those of isd_accept on
 * the same arguments. */
size_t isd_accept_noalloc_max_workspace(void);
int isd_accept_noalloc(const isd_accept_args* args, hipStream_t stream);

/* Block assembly: the stride block of the next step, from the state and
 * outputs isd_accept just wrote (I-DLM page, "Methodologie d'I-DLM >
 * Introspective Strided Decoding (ISD)": one forward carries the clean
 * tokens to verify and MASK positions for the next proposals). Row 0 is
 * the newest emitted token emit[b][n_emit[b] - 1] (not yet in the cache),
 * rows 1..n are the n = st->n_draft[b] pending drafts, the other rows of
 * the 2N are mask_id:
 *   FULL  (n = N-1): [t, d_1 .. d_{N-1}, MASK x N]
 *   FRESH (n = 0):   [t, MASK x (2N-1)]
 * Row i sits at position ctx[b] + i (ctx after the commit).
 *   st        the state isd_accept wrote (n_draft, drafts read)
 *   emit      [C][N], n_emit [C] from the same isd_accept call
 *   ctx       [C]; may be NULL when positions is NULL
 *   tokens    [C][2N] int32 out
 *   positions [C][2N] int32 out, optional (NULL: not written)
 *   is_mask   [C][2N] uint8 out, optional: 1 on MASK rows (the gated LoRA's
 *             mask for the block), 0 elsewhere
 * A sequence whose step was not taken (n_emit outside 1..N) or whose state
 * is neither FULL nor FRESH gets tokens -1, is_mask 0 and ISD_DEV_STATE.
 * Supported: 2 <= N <= 8. Errors: ISD_E_INVALID for a missing pointer.
 */
int isd_block_assemble(const isd_seq_state* st, const int32_t* emit,
                       const int32_t* n_emit, const int32_t* ctx, int C,
                       int N, int32_t mask_id, int32_t* tokens,
                       int32_t* positions, uint8_t* is_mask,
                       int32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------ projections
 * Base projection of the model and the gated LoRA of lossless R-ISD
 * (I-DLM page, "Speedup Factor Explorer" and "Documentation et ressources >
 * Lossless R-ISD": the adapter acts only at MASK positions so clean
 * positions stay bit-identical to the base model).
 *
 * isd_linear: y[M][Nout] = x[M][K] W[Nout][K]^T with bf16 x and W,
 * accumulated in fp32; y is fp32 (ydtype ISD_F32) or the fp32 value rounded
 * to bf16, nearest even (ISD_BF16). Each output's reduction order depends
 * only on K, never on M, on the other rows or on their mask.
 * gated_lora_apply: y[m] += scale * (x[m] A^T) B^T for rows with
 * is_mask[m] != 0; A [r][K] and B [Nout][r] bf16; other rows are never
 * written. U = x A^T (fp32, a split-K GEMM whose split count depends on K
 * only) is built in the workspace, which must hold
 * isd_lora_workspace_size(M, r) bytes (16-byte aligned, owned by the
 * caller). Its first 256 bytes are counters: zero-fill the workspace once
 * before its first use; every call returns them to zero (at any M, r), the
 * rest is scratch. Calls that share a workspace must not overlap in time.
 * isd_linear_gated: y = isd_linear(x, W) then gated_lora_apply, with the
 * delta added in the base GEMM's epilogue; its clean rows equal isd_linear's
 * bit for bit and, with fp32 y, its MASK rows equal those of the two
 * separate calls. With M <= 32 and every workgroup of the call resident on
 * the GPU at once, U is computed by extra workgroups of the GEMM's own
 * launch (one launch instead of two); the bits are the same either way. With bf16 y, gated_lora_apply reads y, adds the delta in
 * fp32 and rounds again, so the separate calls' MASK rows carry a second
 * rounding that the fused call does not.
 * x, W, A, B must be 16-byte aligned, all row-major and contiguous.
 * Supported: K multiple of 64; r multiple of 16, <= 128; ydtype ISD_F32 or
 * ISD_BF16 (y 4- or 2-byte aligned). M == 0 or Nout == 0 returns ISD_OK with
 * nothing launched. Errors: ISD_E_INVALID (null or misaligned pointer,
 * negative size), ISD_E_UNSUPPORTED (K, r, ydtype), and ISD_E_WORKSPACE;
 * nothing is launched on an error.
 */
int isd_linear(const void* x, const void* W, int M, int K, int Nout,
               void* y, int ydtype, hipStream_t stream);
size_t isd_lora_workspace_size(int M, int r);
int gated_lora_apply(const void* x, const void* A, const void* B,
                     const uint8_t* is_mask, int M, int K, int Nout, int r,
                     float scale, void* y, int ydtype, void* ws,
                     size_t ws_bytes, hipStream_t stream);
int isd_linear_gated(const void* x, const void* W, const void* A,
                     const void* B, const uint8_t* is_mask, int M, int K,
                     int Nout, int r, float scale, void* y, int ydtype,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ LM head
 * The distributions the accept step compares are the softmax of the
 * logits the model emits at each row of the block (I-DLM page,
 * "Methodologie d'I-DLM > Entrainement a la coherence introspective": row i
 * gives the distribution of the token at position i + 1; "Documentation et
 * ressources > Inference & ISD": p at clean rows, q at MASK rows). The
 * softmax normaliser of a row is a sum over its vocabulary, so it can be
 * gathered per chunk while the logits are produced, instead of in a second
 * pass over them.
 *
 * isd_lm_head: logits[M][ld] (bf16 bits) = h[M][K] W[V][K]^T, each value
 * the fp32 dot product rounded to nearest even, with the same K-order,
 * M-independent reduction as isd_linear; and chunk_stats[M][nch][2] (fp32,
 * nch = ceil(V / 8192)): for each row and each run of 8192 vocabulary
 * entries, (max, sum of exp(l - max)) of the stored bf16 logits - the
 * statistics isd_accept computes in its first pass. Called with M = C*rows
 * rows in [C][rows] order on a step's block, its outputs feed isd_accept
 * through isd_accept_args.logits and .chunk_stats.
 * ws: isd_lm_head_workspace_size(M, V) bytes, 16-byte aligned, caller-owned,
 * contents on entry ignored (per-row statistics of 128-column tiles).
 * h and W 16-byte aligned, row-major, contiguous; ld >= V.
 * Supported: K multiple of 64. M == 0 returns ISD_OK with nothing launched.
 * Errors: ISD_E_INVALID (null or misaligned pointer, V < 1, ld < V),
 * ISD_E_UNSUPPORTED (K), ISD_E_WORKSPACE; nothing is launched on an error.
 */
size_t isd_lm_head_workspace_size(int M, int V);
int isd_lm_head(const void* h, const void* W, int M, int K, int V,
                void* logits, int64_t ld, float* chunk_stats, void* ws,
                size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------- the decoder block
 * One ISD step is one causal forward of the model (I-DLM page,
 * "Methodologie d'I-DLM"); the released models are built on Qwen3-8B and
 * Qwen3-32B ("Documentation et ressources > Model Zoo"). The pages do not
 * describe the block; these calls are the pieces of the usual pre-norm
 * block of that family (RMSNorm, SwiGLU MLP) that the projections,
 * attention and LM head above do not cover, so that a whole forward runs
 * in this library. Each streams its operands once.
 *
 * isd_rmsnorm: for every row m of h [M][H] (fp32, the residual stream),
 *   h[m] += delta[m] when delta [M][H] is not NULL (the residual add, in
 *   place), then out[m] = bf16(h[m] / sqrt(mean(h[m]^2) + eps) * gamma)
 *   with gamma [H] bf16 and out [M][H] bf16 (round to nearest even). The
 *   mean square is summed in a fixed order per row. H a multiple of 4;
 *   h, delta 16-byte aligned, gamma, out 8-byte aligned.
 * isd_cast_bf16: splits the columns of src [M][ld] fp32 into nparts
 *   (1..4) consecutive ranges of widths[p] columns (host array, each a
 *   multiple of 4) and writes range p, rounded to bf16, to dst[p] (host
 *   array of device pointers, each [M][widths[p]] contiguous, 8-byte
 *   aligned): e.g. a fused Q|K|V projection into q, k and v. ld >= the sum
 *   of the widths and a multiple of 4; src 16-byte aligned.
 * isd_swiglu: out[m][i] = bf16(silu(gu[m][i]) * gu[m][I + i]),
 *   silu(z) = z / (1 + exp(-z)), for gu [M][2I] fp32 (the gate columns,
 *   then the up columns, of one fused projection) and out [M][I] bf16.
 *   I a multiple of 4; gu 16-byte, out 8-byte aligned.
 * Errors: ISD_E_INVALID (null or misaligned pointer, bad size),
 * ISD_E_UNSUPPORTED (H not a multiple of 4); M == 0 launches nothing.
 */
int isd_rmsnorm(float* h, const float* delta, const void* gamma, int M, int H,
                float eps, void* out, hipStream_t stream);
int isd_cast_bf16(const float* src, int64_t ld, int M, int nparts,
                  const int* widths, void* const* dst, hipStream_t stream);
int isd_swiglu(const float* gu, int M, int I, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ISD_H */

// Paged KV write and causal GQA attention of the ISD stride block (gfx950).
//
// The operation: row i of sequence b sits at position ctx_b + i and attends
// causally to positions 0..ctx_b + i of its paged cache; strict causality
// is what lets the model run in an AR serving stack, and the serving kernel
// reads K/V only from pages (I-DLM, fr.news.hada.io, "Methodologie d'I-DLM >
// Serving compatible AR" and "Documentation et ressources > Serving
// (SGLang)").
//
// Kernel design (MI355X-first, not a port of any published kernel):
//  * GQA packing: all (Hq/Hkv) query heads x 2N rows that share one KV head
//    form M <= 128 query columns, processed in blocks of 32 by one wave, so
//    every K/V byte loaded from HBM feeds 32 query rows.
//  * S^T = K . Q^T on MFMA 32x32x16 bf16: a lane owns one query column, so
//    the online-softmax max/sum are lane-local plus one exchange with the
//    lane 32 away. K rows are loaded in a bit-permuted order (bits 2 and 3 of
//    the row swapped) so that the S^T accumulator registers of a lane are
//    exactly the P^T operand of the next product, with no data movement.
//  * O^T = V^T . P^T: the output accumulator also keeps one query column per
//    lane, so the rescale by exp2(m_old - m_new) is a per-lane multiply.
//  * P is split into bf16 hi + lo halves (two MFMAs), keeping about 16
//    mantissa bits on the softmax weights.
//  * Page layout (isd.h) makes every operand a run of 16 contiguous bytes
//    and every 4-lane group a run of 64: K [Hkv][D/8][16 slots][8],
//    V [Hkv][2 half-pages][D][8 slots].
//  * Split-KV: a workgroup holds one wave per (KV head, query block) of a
//    head group; its waves walk the same 32-key tiles (all heads of a page
//    are contiguous). Its share of keys is an equal run of the tiles of all
//    sequences (stream-K) or one fixed-size chunk of one sequence (the
//    batch-invariant split); a sequence cut into several shares leaves
//    (m, l, O) partials that a second kernel merges in share order, so
//    results do not depend on scheduling.
//  * The block's own K/V may come from its rows instead of the pages
//    (isd_attention_with_block): only the boundary tiles read them.
//  * When a KV head has more than 32 query columns (MB > 1 waves per head,
//    bf16), its waves share each K/V tile through LDS: each direct-loads a
//    share of the tile's 1 KB runs, so a K/V byte enters the CU once.
//  * In the chunked split, the chunks of all sequences go to consecutive
//    workgroups, so the XCDs (workgroup id mod 8) get equal counts.
#include "isd_common.hpp"

#include <algorithm>
#include <type_traits>
#include <climits>

namespace isd {

struct AttnParams {
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const void* q;
  const int32_t* ctx;
  void* out;         // [C][rows][Hq][D], fp32, or bf16 bits when obf16
  int obf16;        // outputs rounded to bf16 (nearest even); partials stay fp32
  float* part_o;    // [groups * G][2 slots][HPW * MB][32][D]
  float* part_ml;   // same, [2]: (max, sum)
  int32_t* tile_off;  // [C + 1] tile offsets written for the merge launch
  int32_t* dev_err;
  int table_stride, num_pages;
  int C, rows, Hq, Hkv, group, M;
  int G;             // slices (workgroups) per KV-head group
  int MB, HPW;       // query blocks and KV heads per workgroup (one wave each)
  int CT;            // > 0: batch-invariant split into chunks of CT tiles
  int Kmax;          // chunks per sequence the workspace holds (CT > 0)
  float scale_log2;  // scale * log2(e)
  const void* k_blk;  // optional [C][rows][Hkv][D]: keys at ctx .. ctx+rows-1 come from
  const void* v_blk;  // the block's own K/V rows instead of the pages
};

// K row order inside a 32-key tile: MFMA row i reads tile key pi(i), with
// bits 2 and 3 of i swapped. Then accumulator register e of lane half hh
// holds key 16*(e/8) + 8*hh + e%8, which is the P^T operand layout.
__device__ __forceinline__ int tile_key_of_row(int i) {
  return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}
__device__ __forceinline__ int tile_key_of_reg(int e, int hh) {
  return 16 * (e >> 3) + 8 * hh + (e & 7);
}

template <typename E>
struct AttnOps;

// bfloat16 storage: MFMA 32x32x16, 8 elements per lane per k-step.
template <>
struct AttnOps<uint16_t> {
  static constexpr int kKStep = 16;
  template <int D>
  struct Regs {
    bf16x8 q[D / 16];
    bf16x8 k[D / 16];
    bf16x8 v[D / 32][2];
  };
  static __device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(bf16x8, v);
  }
  // K/V stream through once: non-temporal loads keep them out of the way in
  // the caches (measured about 7% faster than plain loads on this kernel).
  static __device__ __forceinline__ bf16x8 load16_stream(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  }
  static __device__ __forceinline__ bf16x8 zero() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }
  // Loads are unconditional (callers pass pointers that are always inside
  // the buffers: a masked lane or an invalid page reads page 0 or row 0) and
  // a select drops the value: a load under a branch makes the compiler wait
  // for every load in flight at the join, once per load.
  static __device__ __forceinline__ bf16x8 keep(bf16x8 v, bool valid) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    const uint32_t m = valid ? ~0u : 0u;
    return __builtin_bit_cast(bf16x8, u32x4{w[0] & m, w[1] & m, w[2] & m, w[3] & m});
  }

  template <int D>
  static __device__ __forceinline__ void load_q(Regs<D>& r, const uint16_t* qrow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) r.q[s] = keep(load16(qrow + 16 * s + 8 * hh), valid);
  }
  // K operand: lane (row i, half hh) at k-step s holds dims 16s + 8hh .. +8
  // of tile key pi(i).
  template <int D>
  static __device__ __forceinline__ void load_k(Regs<D>& r, const uint16_t* kpage, bool valid, int slot, int hh) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      r.k[s] = keep(load16_stream(kpage + ((2 * s + hh) * 16 + slot) * 8), valid);
  }
  // V^T operand: lane (dim d, half hh) at k-step p (= tile page p) holds
  // slots 8hh .. 8hh+7 of dim d, which the page stores as 16 contiguous
  // bytes right after those of dim d-1 (layout [2][D][8]): every group of
  // four lanes reads 64 contiguous bytes. Keys at or past `limit` are zeroed.
  template <int D>
  static __device__ __forceinline__ void load_v(Regs<D>& r, const uint16_t* vpage, int p, bool valid, int lane32,
                                                int hh, int first_key, int limit) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      const bf16x8 v = keep(load16_stream(vpage + (hh * D + nb * 32 + lane32) * 8), valid);
      // keys at or past limit are cleared without a branch (a branch on the
      // loaded value would make the compiler wait for it right here)
      const int nkeep = limit - first_key;  // keys of this lane's 8 that stay
      u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] &= (2 * k < nkeep ? 0x0000ffffu : 0u) | (2 * k + 1 < nkeep ? 0xffff0000u : 0u);
      r.v[nb][p] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // K operand from a row-major key vector (a block row): the layout of q.
  template <int D>
  static __device__ __forceinline__ void load_k_row(Regs<D>& r, const uint16_t* krow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) r.k[s] = keep(load16(krow + 16 * s + 8 * hh), valid);
  }
  // Keys first_key + j of this lane's run that are block rows (ctx <= key <
  // limit) take their values from vblk (row 0 at vblk, rows `stride` apart).
  // Every load is issued (clamped to a valid row) and selected afterwards,
  // so the 8 * D/32 loads of a lane are in flight together.
  template <int D>
  static __device__ __forceinline__ void patch_v(Regs<D>& r, int p, int lane32, int first_key, int ctx, int limit,
                                                 int rows, const uint16_t* vblk, long stride) {
    uint16_t val[D / 32][8];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        val[nb][j] = vblk[min(max(first_key + j - ctx, 0), rows - 1) * stride + nb * 32 + lane32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      u32x4 w = __builtin_bit_cast(u32x4, r.v[nb][p]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = first_key + j;
        const uint32_t mine = (j & 1) ? 0xffff0000u : 0x0000ffffu;  // element j's bits in its word
        if (key >= ctx && key < limit)
          w[j >> 1] = (w[j >> 1] & ~mine) | (static_cast<uint32_t>(val[nb][j]) << ((j & 1) * 16));
      }
      r.v[nb][p] = __builtin_bit_cast(bf16x8, w);
    }
  }
  template <int D>
  static __device__ __forceinline__ f32x16 qk(const Regs<D>& r) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[s], r.q[s], acc, 0, 0, 0);
    return acc;
  }
  // O^T += V^T . P^T with P split into bf16 hi + lo.
  template <int D>
  static __device__ __forceinline__ void pv(const Regs<D>& r, const float (&p)[16], f32x16 (&o)[D / 32]) {
    bf16x8 hi[2], lo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 wh, wl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float a = p[8 * s + 2 * k], b = p[8 * s + 2 * k + 1];
        uint32_t ua = __float_as_uint(a) & 0xffff0000u, ub = __float_as_uint(b) & 0xffff0000u;
        wh[k] = (ua >> 16) | ub;
        float ra = a - __uint_as_float(ua), rb = b - __uint_as_float(ub);
        wl[k] = f32_to_bf16_bits(ra) | (f32_to_bf16_bits(rb) << 16);
      }
      hi[s] = __builtin_bit_cast(bf16x8, wh);
      lo[s] = __builtin_bit_cast(bf16x8, wl);
    }
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[nb][s], hi[s], o[nb], 0, 0, 0);
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[nb][s], lo[s], o[nb], 0, 0, 0);
      }
    }
  }
};

// fp32 storage: MFMA 32x32x2 f32, one element per lane per k-step.
template <>
struct AttnOps<float> {
  static constexpr int kKStep = 2;
  // as in the bf16 case: unconditional load, then the value is dropped
  static __device__ __forceinline__ float keep(float v, bool valid) {
    return __uint_as_float(__float_as_uint(v) & (valid ? ~0u : 0u));
  }
  template <int D>
  struct Regs {
    float q[D / 2];
    float k[D / 2];
    float v[D / 32][16];
  };
  template <int D>
  static __device__ __forceinline__ void load_q(Regs<D>& r, const float* qrow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 2; ++s) r.q[s] = keep(qrow[2 * s + hh], valid);
  }
  template <int D>
  static __device__ __forceinline__ void load_k(Regs<D>& r, const float* kpage, bool valid, int slot, int hh) {
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
      int d = 2 * s + hh;
      r.k[s] = keep(kpage[((d >> 2) * 16 + slot) * 4 + (d & 3)], valid);
    }
  }
  // V^T operand for k-step e of page p: key 16p + 8hh + e%8.
  template <int D>
  static __device__ __forceinline__ void load_v(Regs<D>& r, const float* vpage, int p, bool valid, int lane32, int hh,
                                                int first_key, int limit) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        bool ok = valid && (first_key + k < limit);
        r.v[nb][8 * p + k] = keep(vpage[(hh * D + nb * 32 + lane32) * 8 + k], ok);
      }
  }
  template <int D>
  static __device__ __forceinline__ void load_k_row(Regs<D>& r, const float* krow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 2; ++s) r.k[s] = keep(krow[2 * s + hh], valid);
  }
  template <int D>
  static __device__ __forceinline__ void patch_v(Regs<D>& r, int p, int lane32, int first_key, int ctx, int limit,
                                                 int rows, const float* vblk, long stride) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = first_key + j;
        const float val = vblk[min(max(key - ctx, 0), rows - 1) * stride + nb * 32 + lane32];
        if (key >= ctx && key < limit) r.v[nb][8 * p + j] = val;
      }
  }
  template <int D>
  static __device__ __forceinline__ f32x16 qk(const Regs<D>& r) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 2; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(r.k[s], r.q[s], acc, 0, 0, 0);
    return acc;
  }
  template <int D>
  static __device__ __forceinline__ void pv(const Regs<D>& r, const float (&p)[16], f32x16 (&o)[D / 32]) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(r.v[nb][e], p[e], o[nb], 0, 0, 0);
  }
};

constexpr int kMaxSeqs = 8192;   // sequences per attention call (LDS prefix sums)
constexpr int kTileBatch = 1024;  // tiles whose page ids are staged in LDS at once
constexpr int kMaxChunkTiles = 1 << 16;  // largest chunk of the batch-invariant split

template <typename E, int D>
__device__ __forceinline__ const E* page_ptr(const void* pool, int pid, int Hkv, int g) {
  return static_cast<const E*>(pool) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16);
}

// Work split ("stream-K"): the tiles (32 keys) of all sequences are laid
// end to end, tiles(b) = ceil((ctx_b + rows) / 32), and slice w of G takes
// tiles [floor(w*T/G), floor((w+1)*T/G)) of that list, so every workgroup
// streams the same number of bytes however ragged the contexts are. A
// workgroup holds HPW KV heads x MB query blocks, one wave each; its waves
// walk the same pages together (all heads of a page are contiguous). A
// sequence that lies wholly inside one slice is finalised in registers; the
// pieces of a sequence shared by several slices are written to two partial
// slots per slice (its first and its last sequence) and merged afterwards in
// slice order, so results do not depend on scheduling.
//
// Batch-invariant split (CT > 0): each sequence is cut at fixed multiples of
// CT tiles from position 0, and each chunk gets a workgroup of its own.
// Pieces, their order and the merge then depend only on the sequence
// itself, and a query column's arithmetic depends only on its own keys:
// masked keys add exact zeros (exp2 of -inf), a rescale of a column
// whose maximum did not move multiplies by exp2(0) = 1, and the MFMA result
// of one column does not depend on the others. So a row of a block of rows
// comes out bit for bit equal to the same query sent alone with ctx + row
// cached tokens (the autoregressive forward), whatever else is in the batch.
// Cache-policy operand of a direct-to-LDS load: non-temporal (the K/V
// stream through once, as the register loads' non-temporal hint says).
constexpr int kNonTemporal = 2;

// Wait until this wave's vector-memory operations (vm = 0) or its LDS
// operations (lgkm = 0) are done; the exp counter is not waited on.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier with no memory fence (the waits it needs are explicit);
// the empty asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive prefix sum of count(b) over the C sequences into s_off[0..C]
// (s_off[C] = total), by all `nthreads` threads of the workgroup: each sums
// a run of sequences, a scan inside each wave, then the totals of the waves
// before (integer adds, so the order is free). count is called twice per
// sequence; `visit(b)` runs once per sequence, on the thread that owns it.
template <typename Count, typename Visit>
__device__ __forceinline__ void prefix_over_sequences(int C, int nthreads, int* s_off, int* s_part, Count count,
                                                      Visit visit) {
  const int per = (C + nthreads - 1) / nthreads;
  const int b0 = threadIdx.x * per;
  int sum = 0;
  for (int b = b0; b < min(C, b0 + per); ++b) sum += count(b);
  const int ln = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (ln >= d) incl += v;
  }
  if (ln == kWave - 1) s_part[wv] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w2 = 0; w2 < wv; ++w2) run += s_part[w2];
  for (int b = b0; b < min(C, b0 + per); ++b) {
    s_off[b] = run;
    visit(b);
    run += count(b);
  }
  if (b0 < C && min(C, b0 + per) == C) s_off[C] = run;
  __syncthreads();
}

// Largest b in [0, C) with s_off[b] <= x (x < s_off[C]): the sequence whose
// range of the prefix holds x (sequences with an empty range are skipped).
__device__ __forceinline__ int sequence_holding(const int* s_off, int C, long x) {
  int lo = 0, hi = C - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename E, int D, bool kChunked, bool kShare>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnParams p) {
  using Ops = AttnOps<E>;
  const int MB = p.MB;
  const int G = p.G;
  const int hg = blockIdx.x / G;
  const int w = blockIdx.x % G;
  const int nthreads = 64 * p.HPW * MB;

  // Prefix over the sequences: tile offsets (stream-K split) or chunk
  // offsets (chunked split).
  __shared__ int s_off[kMaxSeqs + 1];
  __shared__ int s_part[512 / kWave];  // per-wave totals of the prefix sum
  __shared__ int s_pid[2 * kTileBatch];  // page ids of the current tile batch
  // K/V tile of each KV head shared by its MB > 1 query-block waves (bf16):
  // D / 8 slots of 1 KB (64 lanes x 16 bytes), K runs first, then the V runs
  // of the tile's two pages.
  constexpr int kSlotsK = D / 16, kSlots = D / 8;
  // (kShare: bf16 with MB > 1, so HPW <= 8 / MB <= 4 heads)
  static_assert(!kShare || std::is_same<E, uint16_t>::value, "shared tiles are bf16");
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[kShare ? 4 * kSlots * 512 : 8];
  int t_begin = 0, t_end = 0;
  int u_first = 0;                   // first sequence of this workgroup
  int c_nt = 0, c_units = 0, c_k = 0;  // chunked split: tiles, chunks, this chunk
  if constexpr (kChunked) {
    // The chunks of all sequences, in sequence order, go to consecutive
    // workgroups of the head group (workgroup w takes the w-th); the
    // workgroups past the last chunk leave at once. Consecutive ids are
    // spread over the XCDs in turn, so every XCD gets an equal count of
    // chunks, and as long as there are no more chunks than CUs they all run
    // in one round. A sequence flagged bad (ctx < 0, or ctx + rows beyond the
    // chunks the workspace holds) has no chunks.
    auto units_of = [&](int b) {
      const int ctx = p.ctx[b];
      if (ctx < 0) return 0;
      const int u = ((ctx + p.rows + 31) / 32 + p.CT - 1) / p.CT;
      return u > p.Kmax ? 0 : u;
    };
    prefix_over_sequences(p.C, nthreads, s_off, s_part, units_of, [&](int b) {
      if (w != 0 || hg != 0) return;
      const int ctx = p.ctx[b];
      if (ctx < 0) set_dev_err(p.dev_err, ISD_DEV_STATE);
      else if (((ctx + p.rows + 31) / 32 + p.CT - 1) / p.CT > p.Kmax) set_dev_err(p.dev_err, ISD_DEV_CAPACITY);
    });
    if (w >= s_off[p.C]) return;
    u_first = sequence_holding(s_off, p.C, w);
    c_k = w - s_off[u_first];
    c_nt = (p.ctx[u_first] + p.rows + 31) / 32;
    c_units = (c_nt + p.CT - 1) / p.CT;
  } else {
    prefix_over_sequences(
        p.C, nthreads, s_off, s_part,
        [&](int b) {
          const int ctx = p.ctx[b];
          return ctx < 0 ? 0 : (ctx + p.rows + 31) / 32;
        },
        [&](int b) {
          if (p.ctx[b] < 0 && w == 0 && hg == 0) set_dev_err(p.dev_err, ISD_DEV_STATE);
        });
    const long T = s_off[p.C];
    t_begin = static_cast<int>(w * T / G);
    t_end = static_cast<int>((w + 1) * T / G);
    if (w == 0 && hg == 0)  // the merge launch reads the offsets back
      for (int b = threadIdx.x; b <= p.C; b += nthreads) p.tile_off[b] = s_off[b];
    if (t_begin >= t_end) return;
    u_first = sequence_holding(s_off, p.C, t_begin);
  }

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int lane32 = lane & 31;
  const int hh = lane >> 5;
  const int rb = wave % MB;
  const int hl_w = wave / MB;
  const int g = hg * p.HPW + hl_w;
  const int qi = rb * 32 + lane32;  // query column of this lane
  const bool qvalid = qi < p.M;
  const int hl = qvalid ? qi / p.rows : 0;
  const int irow = qvalid ? qi % p.rows : p.rows - 1;
  const int h = g * p.group + hl;
  const int krow_key = tile_key_of_row(lane32);  // tile key this lane loads for K
  const int kpg = krow_key >> 4;
  const int kslot = krow_key & 15;
  uint32_t err = 0;

  typename Ops::template Regs<D> r;
  f32x16 o[D / 32];
  float m_run, l_run;

  // Pieces: the slice's share of each sequence it touches (stream-K), or
  // the workgroup's one chunk (chunked split).
  for (int b = u_first; kChunked ? b == u_first : (b < p.C && s_off[b] < t_end); ++b) {
    int nt, k = 0, tb0 = 0;
    if constexpr (kChunked) {
      nt = c_nt;
      k = c_k;
    } else {
      tb0 = s_off[b];
      nt = s_off[b + 1] - tb0;
    }
    const int lt0 = kChunked ? k * p.CT : max(t_begin, tb0) - tb0;
    const int lt1 = kChunked ? min(nt, lt0 + p.CT) : min(t_end, tb0 + nt) - tb0;
    if (lt0 >= lt1) continue;
    const int ctx = p.ctx[b];
    const int L = ctx + p.rows;  // positions 0 .. L-1 are read
    const bool blk = p.k_blk != nullptr;  // keys ctx .. L-1 from the block rows
    const int page_end = blk ? ctx : L;   // positions read from pages
    const int vis_limit = ctx + irow;
    const int32_t* table = p.block_table + static_cast<size_t>(b) * p.table_stride;

    const E* qrow = static_cast<const E*>(p.q) + ((static_cast<size_t>(b) * p.rows + irow) * p.Hq + h) * D;
    Ops::template load_q<D>(r, qrow, qvalid, hh);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] = f32x16{};
    m_run = -1e30f;  // finite floor: exp2(m_old - m_new) stays defined
    l_run = 0.f;

    auto clamp_pid = [&](int pid) {
      if (pid < 0 || pid >= p.num_pages) {
        err |= ISD_DEV_PAGE_OOB;
        return 0;
      }
      return pid;
    };
    // online-softmax update and PV product for one tile of scores
    auto consume = [&](const f32x16& s, int t0, bool masked) {
      float sv[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[e];
        if (masked) x = (t0 + tile_key_of_reg(e, hh) <= vis_limit) ? x : -INFINITY;
        sv[e] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run, tmax * p.scale_log2);
      float pr[16];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pr[e] = fast_exp2(fmaf(sv[e], p.scale_log2, -m_new));
        psum += pr[e];
      }
      if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {  // some row maximum grew
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[nb][e] *= alpha;
      }
      m_run = m_new;
      l_run += psum;
      Ops::template pv<D>(r, pr, o);
    };

    // The piece's page ids are staged in LDS a batch at a time (one
    // cooperative load), so no tile waits on a block-table round trip
    // before it can issue its K/V loads.
    const int full_end = min(lt1, max(0, min(blk ? ctx : ctx + 1, p.table_stride * 16) / 32));
    for (int bt0 = lt0; bt0 < lt1; bt0 += kTileBatch) {
      const int bt1 = min(lt1, bt0 + kTileBatch);
      __syncthreads();  // the previous batch is no longer read
      for (int i = threadIdx.x; i < 2 * (bt1 - bt0); i += nthreads) {
        const int col = 2 * bt0 + i;
        s_pid[i] = col < p.table_stride ? table[col] : -1;
      }
      __syncthreads();

      // Full tiles (all 32 keys visible to every row, pages inside the
      // table) run a straight-line, software-pipelined loop: the K loads of
      // the next tile are issued as soon as QK^T has consumed the K
      // registers, the V loads right after PV.
      const int fe = min(bt1, full_end);
      int lt = bt0;
      if (lt < fe) {
        const E* kpage;
        const E* vpage0;
        const E* vpage1;
        auto pages = [&](int tl) {
          const int pid0 = clamp_pid(s_pid[2 * (tl - bt0)]), pid1 = clamp_pid(s_pid[2 * (tl - bt0) + 1]);
          kpage = page_ptr<E, D>(p.k_pages, kpg ? pid1 : pid0, p.Hkv, g);
          vpage0 = page_ptr<E, D>(p.v_pages, pid0, p.Hkv, g);
          vpage1 = page_ptr<E, D>(p.v_pages, pid1, p.Hkv, g);
        };
        if constexpr (kShare) {
          // The MB waves of a KV head (one per query block) need the same
          // K/V tile. Each loads every MB-th of its 1 KB slots straight into
          // LDS; after a barrier all of them read the whole tile from there,
          // so each K/V byte enters the CU once instead of MB times (a CU
          // streams unique bytes about 1.4x faster than bytes it fetches
          // twice). The next tile's loads are issued once every wave has read
          // this one, one tile ahead of use like the loop below.
          {
            uint16_t* const tile = s_tile + hl_w * (kSlots * 512);
            auto issue = [&](int tl) {
              pages(tl);
#pragma unroll
              for (int i = 0; i < kSlots; ++i) {
                if (i % MB != rb) continue;  // wave-uniform
                const uint16_t* src;
                if (i < kSlotsK) {
                  src = kpage + ((2 * i + hh) * 16 + kslot) * 8;
                } else {
                  const int j = i - kSlotsK, pg = j / (D / 32), nb = j % (D / 32);
                  src = (pg ? vpage1 : vpage0) + (hh * D + nb * 32 + lane32) * 8;
                }
                __builtin_amdgcn_global_load_lds(src, tile + i * 512, 16, 0, kNonTemporal);
              }
            };
            issue(lt);
            for (;;) {
              const bool more = lt + 1 < fe;
              wait_vm0();  // this wave's share of tile lt is in LDS
              plain_barrier();
#pragma unroll
              for (int i = 0; i < kSlots; ++i) {
                const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + i * 512 + 8 * lane));
                if (i < kSlotsK) r.k[i] = v;
                else r.v[(i - kSlotsK) % (D / 32)][(i - kSlotsK) / (D / 32)] = v;
              }
              wait_lgkm0();  // every wave holds tile lt in registers before
              plain_barrier();  // the next tile's loads overwrite it
              if (more) issue(lt + 1);
              consume(Ops::template qk<D>(r), 32 * lt, false);
              ++lt;
              if (!more) break;
            }
          }
        }
        if constexpr (!kShare) {
        pages(lt);
        Ops::template load_k<D>(r, kpage, true, kslot, hh);
        Ops::template load_v<D>(r, vpage0, 0, true, lane32, hh, 0, INT_MAX);
        Ops::template load_v<D>(r, vpage1, 1, true, lane32, hh, 0, INT_MAX);
        for (;;) {
          const bool more = lt + 1 < fe;
          pages(more ? lt + 1 : lt);  // past the end: reload this tile, unused
          const f32x16 sc = Ops::template qk<D>(r);
          Ops::template load_k<D>(r, kpage, true, kslot, hh);
          // Keep the prefetches where they are: without these barriers the
          // compiler sinks them next to their use and the load latency is
          // exposed on every tile.
          asm volatile("" ::: "memory");
          consume(sc, 32 * lt, false);
          Ops::template load_v<D>(r, vpage0, 0, true, lane32, hh, 0, INT_MAX);
          Ops::template load_v<D>(r, vpage1, 1, true, lane32, hh, 0, INT_MAX);
          asm volatile("" ::: "memory");
          ++lt;
          // Keep the waves in step. Two waves share a SIMD and the older one
          // wins issue, so without this the first four heads finish far
          // ahead and the tail of the piece runs on half the waves (measured
          // 60 us of a 240 us launch). Every wave runs the same tiles, so
          // the barrier count is uniform; it needs no memory fence.
          if ((lt & 3) == 0) __builtin_amdgcn_s_barrier();
          if (!more) break;
        }
        }
      }
      for (; lt < bt1; ++lt) {  // boundary tiles: causal mask, positions past L, table end
        const int t0 = 32 * lt;
        const E* kp[2];
        const E* vp[2];
        bool ok[2];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const int first = t0 + 16 * pg;
          bool valid = first < page_end;
          int pid = 0;
          if (valid) {
            if ((first >> 4) >= p.table_stride) {
              err |= ISD_DEV_CAPACITY;
              valid = false;
            } else {
              pid = s_pid[2 * (lt - bt0) + pg];
              if (pid < 0 || pid >= p.num_pages) {
                err |= ISD_DEV_PAGE_OOB;
                valid = false;
                pid = 0;
              }
            }
          }
          ok[pg] = valid;
          kp[pg] = page_ptr<E, D>(p.k_pages, pid, p.Hkv, g);
          vp[pg] = page_ptr<E, D>(p.v_pages, pid, p.Hkv, g);
        }
        const int kpos = t0 + krow_key;  // this lane's key
        if (blk && kpos >= ctx) {
          const E* krow = static_cast<const E*>(p.k_blk) +
                          ((static_cast<size_t>(b) * p.rows + min(kpos - ctx, p.rows - 1)) * p.Hkv + g) * D;
          Ops::template load_k_row<D>(r, krow, kpos < L, hh);
        } else {
          Ops::template load_k<D>(r, kpg ? kp[1] : kp[0], kpg ? ok[1] : ok[0], kslot, hh);
        }
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          Ops::template load_v<D>(r, vp[pg], pg, ok[pg], lane32, hh, t0 + 16 * pg + 8 * hh, L);
          if (blk)
            Ops::template patch_v<D>(r, pg, lane32, t0 + 16 * pg + 8 * hh, ctx, L, p.rows,
                                     static_cast<const E*>(p.v_blk) + (static_cast<size_t>(b) * p.rows * p.Hkv + g) * D,
                                     static_cast<long>(p.Hkv) * D);
        }
        consume(Ops::template qk<D>(r), t0, true);
      }
    }

    // Finalise this (sequence, head, query block) piece. Register e of
    // block nb holds dim 32nb + 8(e/4) + 4hh + e%4: four registers make one
    // 16-byte store.
    const float l_tot = l_run + shfl_xor_f(l_run, 32);
    const bool whole = kChunked ? c_units == 1 : lt0 == 0 && lt1 == nt;
    if (qvalid) {
      float* dst = nullptr;
      float mul;
      const size_t oidx = ((static_cast<size_t>(b) * p.rows + irow) * p.Hq + h) * D;
      if (whole) {
        if (!p.obf16) dst = static_cast<float*>(p.out) + oidx;
        mul = 1.f / l_tot;
      } else {
        // partial piece of this wave's query columns
        const size_t pidx =
            kChunked ? ((static_cast<size_t>(b) * p.Kmax + k) * (p.Hkv / p.HPW) + hg) * (p.HPW * MB) + hl_w * MB + rb
                     : (static_cast<size_t>(hg * G + w) * 2 + (b == u_first ? 0 : 1)) * (p.HPW * MB) + hl_w * MB + rb;
        const size_t idx = pidx * 32 + lane32;
        dst = p.part_o + idx * D;
        mul = 1.f;
        if (hh == 0) {
          p.part_ml[idx * 2] = m_run;
          p.part_ml[idx * 2 + 1] = l_tot;
        }
      }
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[nb][4 * q4 + e] * mul;
          if (dst) {
            *reinterpret_cast<f32x4*>(dst + nb * 32 + 8 * q4 + 4 * hh) = v;
          } else {  // a whole piece into bf16 outputs: four values, one 8-byte store
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + oidx + nb * 32 + 8 * q4 + 4 * hh) =
                make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                           f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
          }
        }
    }
  }
  if (err) set_dev_err(p.dev_err, err);
}

// Log-sum-exp merge of the pieces of one (sequence, KV head, query block)
// held by several slices, in slice order (an online rescale, so the pieces
// are read once). A workgroup takes 32 dims of the block's 32 query
// columns: thread t owns column t/8 and one float4 of dims; the (max, sum)
// and vectors of up to sixteen pieces are loaded together before any is
// combined. Every thread of a column runs the same (max, sum) recurrence,
// so how the dims are spread over threads does not change any value.
template <int D>
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnParams p) {
  const int MB = p.MB;
  const int b = blockIdx.x / p.Hkv;
  const int g = blockIdx.x % p.Hkv;
  const int qb = blockIdx.y / (D / 32);
  const int G = p.G;
  const int hg = g / p.HPW, hl_w = g % p.HPW;
  // Pieces j = 0 .. n-1 of the sequence, in order: its slices wa .. wb
  // (stream-K split) or its chunks (chunked split).
  long T = 0;
  int tb0 = 0, wa = 0, n;
  if (p.CT > 0) {
    const int ctx = p.ctx[b];
    if (ctx < 0) return;
    n = ((ctx + p.rows + 31) / 32 + p.CT - 1) / p.CT;
    if (n > p.Kmax) return;  // not computed (flagged by the main launch)
  } else {
    T = p.tile_off[p.C];
    tb0 = p.tile_off[b];
    const int tb1 = p.tile_off[b + 1];
    if (tb1 <= tb0 || T == 0) return;
    // slice holding tile x: the largest w with floor(w*T/G) <= x
    auto slice_of = [&](long x) { return static_cast<int>(((x + 1) * G + T - 1) / T - 1); };
    wa = slice_of(tb0);
    n = slice_of(tb1 - 1) - wa + 1;
  }
  if (n == 1) return;  // finalised by the main launch
  constexpr int kDimsPerThread = 4;
  constexpr int kV = kDimsPerThread / 4;
  constexpr int kBatch = 16;
  const int col = qb * 32 + threadIdx.x / (256 / 32);
  const int d0 = (blockIdx.y % (D / 32)) * 32 + (threadIdx.x % (256 / 32)) * kDimsPerThread;
  if (col >= p.M) return;
  auto piece = [&](int j) {
    size_t pidx;
    if (p.CT > 0) {
      pidx = ((static_cast<size_t>(b) * p.Kmax + j) * (p.Hkv / p.HPW) + hg) * (p.HPW * MB) + hl_w * MB + qb;
    } else {
      const int w2 = wa + j;
      const int slot = (w2 * T / G) >= tb0 ? 0 : 1;
      pidx = (static_cast<size_t>(hg * G + w2) * 2 + slot) * (p.HPW * MB) + hl_w * MB + qb;
    }
    return pidx * 32 + (col - qb * 32);
  };
  // a slice whose range is empty (more slices than tiles) holds no piece
  auto empty = [&](int j) { return p.CT <= 0 && ((wa + j) * T / G) == ((wa + j + 1) * T / G); };
  float m_run = -1e30f, l_run = 0.f;  // finite floor: exp2(m_run - m_new) stays defined
  f32x4 acc[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  // batches of B pieces, B the smallest of 2, 4, 8, 16 that holds n (the
  // same arithmetic for every B: one online step per piece, in order)
  auto merge_all = [&](auto batch) {
    constexpr int B = decltype(batch)::value;
    for (int j0 = 0; j0 < n; j0 += B) {
      float mv[B], lv[B];
      f32x4 ov[B][kV];
      bool has[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        has[j] = j0 + j < n && !empty(j0 + j);
        const size_t idx = piece(has[j] ? j0 + j : 0);  // piece 0 always exists
        mv[j] = p.part_ml[idx * 2];
        lv[j] = p.part_ml[idx * 2 + 1];
        const f32x4* src = reinterpret_cast<const f32x4*>(p.part_o + idx * D + d0);
#pragma unroll
        for (int k = 0; k < kV; ++k) ov[j][k] = src[k];
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (!has[j]) continue;
        const float m_new = fmaxf(m_run, mv[j]);
        const float a = fast_exp2(m_run - m_new), c = fast_exp2(mv[j] - m_new);
        l_run = fmaf(l_run, a, lv[j] * c);
#pragma unroll
        for (int k = 0; k < kV; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[k][e] = fmaf(acc[k][e], a, ov[j][k][e] * c);
        m_run = m_new;
      }
    }
  };
  if (n <= 2) merge_all(std::integral_constant<int, 2>{});
  else if (n <= 4) merge_all(std::integral_constant<int, 4>{});
  else if (n <= 8) merge_all(std::integral_constant<int, 8>{});
  else merge_all(std::integral_constant<int, kBatch>{});
  const int hl = col / p.rows, i = col % p.rows;
  const int h = g * p.group + hl;
  const size_t oidx = ((static_cast<size_t>(b) * p.rows + i) * p.Hq + h) * D + d0;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    f32x4 v = acc[k];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = v[e] * inv;
    if (p.obf16)
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + oidx)[k] =
          make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                     f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
    else
      reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + oidx)[k] = v;
  }
}

// ----------------------------------------------------------------- KV write
template <typename E, int D>
__global__ __launch_bounds__(256) void kv_write_kernel(void* k_pages, void* v_pages, const int32_t* block_table,
                                                       int table_stride, int num_pages, int Hkv, const E* k,
                                                       const E* v, const int32_t* pos0, const int32_t* nrows, int C,
                                                       int rows, int32_t* dev_err, long layer_pool,
                                                       long layer_rows, int k_blocks, int v_units) {
  constexpr int KP = Elem<E>::kPerVec;
  // grid (blocks, sequences, layers): b is uniform, so its position and row
  // count come in through scalar loads; layer z has its pools layer_pool
  // elements and its rows layer_rows elements on.
  k_pages = static_cast<E*>(k_pages) + blockIdx.z * layer_pool;
  v_pages = static_cast<E*>(v_pages) + blockIdx.z * layer_pool;
  k += blockIdx.z * layer_rows;
  v += blockIdx.z * layer_rows;
  const int b = blockIdx.y;
  const int nr = nrows ? min(nrows[b], rows) : rows;
  const int p0 = pos0[b];
  if (static_cast<int>(blockIdx.x) < k_blocks) {
    // K: one thread per (row, head, 16-byte run); a row's run is whole in
    // the page ([D/KP][16 slots][KP]). Rows past nrows leave before loading.
    const int per_row = Hkv * (D / KP);
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * per_row) return;
    const int r = idx / per_row;
    if (r >= nr) return;
    const int c = idx % (D / KP);
    const int g = (idx / (D / KP)) % Hkv;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k + ((static_cast<size_t>(b) * rows + r) * Hkv + g) * D + c * KP);
    const int pos = p0 + r;
    if (pos < 0) {
      set_dev_err(dev_err, ISD_DEV_STATE);
      return;
    }
    const int col = pos >> 4, slot = pos & 15;
    if (col >= table_stride) {
      set_dev_err(dev_err, ISD_DEV_CAPACITY);
      return;
    }
    const int pid = block_table[static_cast<size_t>(b) * table_stride + col];
    if (pid < 0 || pid >= num_pages) {
      set_dev_err(dev_err, ISD_DEV_PAGE_OOB);
      return;
    }
    E* kpage = static_cast<E*>(k_pages) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16);
    *reinterpret_cast<u32x4*>(kpage + (c * 16 + slot) * KP) = kv;
    return;
  }
  // V: the page keeps the 8 slots of a half page contiguous per dimension
  // ([2 halves][D][8 slots]), so one thread per (half page, head, dimension)
  // rewrites that 8-slot run whole: it reads it, replaces the slots of the
  // rows being written and stores it back (whole runs instead of 2-byte
  // scatters). Unit u is the (u+1)-th half page from the one holding pos0.
  // Positions the K threads flag (negative, past the table, bad page) are
  // skipped here; slots of other positions keep their values. Two sequences
  // must not write into one page in the same call.
  const int idx = (blockIdx.x - k_blocks) * blockDim.x + threadIdx.x;
  const int d = idx % D;
  const int g = (idx / D) % Hkv;
  const int u = idx / (D * Hkv);
  if (u >= v_units) return;
  const int first = ((p0 >> 3) + u) * 8;  // first position of the half page
  const int lo = max(max(p0, first), 0), hi = min(p0 + nr, first + 8);
  if (lo >= hi) return;
  const int col = first >> 4;
  if (col >= table_stride) return;
  const int pid = block_table[static_cast<size_t>(b) * table_stride + col];
  if (pid < 0 || pid >= num_pages) return;
  E* run = static_cast<E*>(v_pages) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16) + (((first >> 3) & 1) * D + d) * 8;
  constexpr int kVecs = 8 * static_cast<int>(sizeof(E)) / 16;
  u32x4 w[kVecs];
#pragma unroll
  for (int i = 0; i < kVecs; ++i) w[i] = reinterpret_cast<const u32x4*>(run)[i];
  E* ev = reinterpret_cast<E*>(w);
  const E* vrow = v + (static_cast<size_t>(b) * rows * Hkv + g) * D + d;  // row 0 of this head and dimension
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = first + j;
    if (pos >= lo && pos < hi) ev[j] = vrow[static_cast<size_t>(pos - p0) * Hkv * D];
  }
#pragma unroll
  for (int i = 0; i < kVecs; ++i) reinterpret_cast<u32x4*>(run)[i] = w[i];
}

}  // namespace isd

// ================================================================ host API
namespace {

using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_kv(const isd_kv_cache* kv) {
  if (!kv || !kv->k_pages || !kv->v_pages || !kv->block_table) return ISD_E_INVALID;
  if (kv->page_size != ISD_PAGE_SIZE) return ISD_E_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return ISD_E_UNSUPPORTED;
  if (kv->dtype != ISD_BF16 && kv->dtype != ISD_F32) return ISD_E_UNSUPPORTED;
  if (kv->num_kv_heads < 1 || kv->num_kv_heads > 64) return ISD_E_UNSUPPORTED;
  if (kv->num_pages < 1 || kv->table_stride < 1) return ISD_E_INVALID;
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages)) return ISD_E_INVALID;
  return ISD_OK;
}

struct AttnPlan {
  int MB, HPW, groups, G;
  int CT, Kmax;  // batch-invariant split (CT > 0): chunk tiles, chunks per sequence
  size_t off_bytes, part_o_bytes, part_ml_bytes;
  size_t total() const { return off_bytes + part_o_bytes + part_ml_bytes; }
};

int plan_attention(int C, int rows, int Hq, const isd_kv_cache* kv, int max_len, int slices, AttnPlan* plan) {
  if (C < 0 || rows < 1 || rows > 64 || Hq < 1) return ISD_E_INVALID;
  if (C > kMaxSeqs) return ISD_E_UNSUPPORTED;
  const int Hkv = kv->num_kv_heads;
  if (Hq % Hkv != 0) return ISD_E_UNSUPPORTED;
  const int M = (Hq / Hkv) * rows;
  if (M > 128) return ISD_E_UNSUPPORTED;
  if (max_len < rows) return ISD_E_INVALID;
  if (slices < -kMaxChunkTiles) return ISD_E_INVALID;
  plan->MB = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  // KV heads per workgroup: the largest power of two that divides Hkv with
  // at most 8 waves (one per head and query block) in the workgroup.
  plan->HPW = 1;
  while (plan->HPW * 2 * plan->MB <= 8 && Hkv % (plan->HPW * 2) == 0) plan->HPW *= 2;
  plan->groups = Hkv / plan->HPW;
  // Default: 1536 waves, spread over the head groups: a full workgroup (8
  // waves, the register-file limit of this kernel) on three CUs in four.
  // Fewer slices cut the partials (two per slice) and measured faster than
  // one workgroup per CU on ragged 1K-8K contexts (234 vs 245 us per call at
  // 8B shapes, C = 64). Never more slices than tiles.
  const long auto_G = std::max(1, 1536 / (plan->HPW * plan->MB) / plan->groups);
  const long max_tiles = static_cast<long>(C) * ((max_len + 31) / 32);
  size_t pieces;  // partial (query block, KV head) pieces the workspace holds
  if (slices < 0) {
    // batch-invariant split: one workgroup per (head group, sequence, chunk
    // of CT tiles), so the hardware dispatcher balances the chunks
    plan->CT = -slices;
    plan->Kmax = static_cast<int>(((max_len + 31) / 32 + plan->CT - 1) / plan->CT);
    const long G = static_cast<long>(C) * plan->Kmax;
    if (G * Hkv > INT_MAX) return ISD_E_UNSUPPORTED;  // grid size
    plan->G = static_cast<int>(std::max(1L, G));
    pieces = static_cast<size_t>(C) * plan->Kmax;
  } else {
    plan->CT = 0;
    plan->Kmax = 0;
    long G = slices ? slices : auto_G;
    if (G > max_tiles) G = std::max(1L, max_tiles);
    plan->G = static_cast<int>(G);
    pieces = static_cast<size_t>(plan->G) * 2;
  }
  pieces *= static_cast<size_t>(plan->groups) * plan->HPW * plan->MB * 32;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  plan->off_bytes = up(static_cast<size_t>(C + 1) * sizeof(int32_t));
  plan->part_o_bytes = up(pieces * kv->head_dim * sizeof(float));
  plan->part_ml_bytes = up(pieces * 2 * sizeof(float));
  return ISD_OK;
}

template <typename E, int D>
hipError_t launch_attention_typed(const AttnParams& p, int groups, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(groups * p.G)), block(static_cast<unsigned>(64 * p.HPW * p.MB));
  // bf16 heads with several query-block waves share each K/V tile through LDS
  const bool share = std::is_same<E, uint16_t>::value && p.MB > 1;
  if (p.CT > 0) {
    if (share) hipLaunchKernelGGL((attention_kernel<E, D, true, std::is_same<E, uint16_t>::value>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attention_kernel<E, D, true, false>), grid, block, 0, stream, p);
  } else {
    if (share) hipLaunchKernelGGL((attention_kernel<E, D, false, std::is_same<E, uint16_t>::value>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attention_kernel<E, D, false, false>), grid, block, 0, stream, p);
  }
  hipLaunchKernelGGL((attention_merge_kernel<D>),
                     dim3(static_cast<unsigned>(p.C * p.Hkv), static_cast<unsigned>(p.MB * (D / 32))), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

// the bodies of isd_attention / isd_attention_with_block and of
// isd_kv_write / isd_kv_write_layers
int attention_call(const isd_kv_cache* kv, const void* k_blk, const void* v_blk, const void* q, const int32_t* ctx,
                   int C, int rows, int num_q_heads, float scale, int max_len, int slices, void* out, int odtype,
                   void* ws, size_t ws_bytes, int32_t* dev_err, hipStream_t stream);

int kv_write_call(const isd_kv_cache* kv, int layers, int64_t layer_stride, const void* k, const void* v,
                  const int32_t* pos0, const int32_t* nrows, int C, int rows, int32_t* dev_err, hipStream_t stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  if (C < 0 || rows < 0) return ISD_E_INVALID;
  if (C == 0 || rows == 0) return ISD_OK;
  if (C > 65535) return ISD_E_UNSUPPORTED;  // sequences map to a grid dimension
  if (!k || !v || !pos0) return ISD_E_INVALID;
  if (!aligned16(k) || !aligned16(v)) return ISD_E_INVALID;
  rc = isd_check_device_internal();
  if (rc) return rc;
  const int D = kv->head_dim;
  const int KP = kv->dtype == ISD_BF16 ? 8 : 4;
  const long per_seq = static_cast<long>(rows) * kv->num_kv_heads * (D / KP);
  const long layer_rows = static_cast<long>(C) * rows * kv->num_kv_heads * D;
  // K blocks first, then V blocks: `rows` consecutive positions touch at
  // most (rows + 7) / 8 + 1 half pages
  const int k_blocks = static_cast<int>((per_seq + 255) / 256);
  const int v_units = (rows + 7) / 8 + 1;
  const long v_threads = static_cast<long>(v_units) * kv->num_kv_heads * D;
  const long blocks = k_blocks + (v_threads + 255) / 256;
  if (blocks > INT_MAX) return ISD_E_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(C), static_cast<unsigned>(layers));
#define ISD_KVW(E, DD)                                                                                          \
  hipLaunchKernelGGL((kv_write_kernel<E, DD>), grid, dim3(256), 0, stream, kv->k_pages, kv->v_pages,            \
                     kv->block_table, kv->table_stride, kv->num_pages, kv->num_kv_heads, static_cast<const E*>(k), \
                     static_cast<const E*>(v), pos0, nrows, C, rows, dev_err, static_cast<long>(layer_stride),    \
                     layer_rows, k_blocks, v_units)
  if (kv->dtype == ISD_BF16) {
    if (D == 128) ISD_KVW(uint16_t, 128);
    else ISD_KVW(uint16_t, 64);
  } else {
    if (D == 128) ISD_KVW(float, 128);
    else ISD_KVW(float, 64);
  }
#undef ISD_KVW
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // namespace

extern "C" {

size_t isd_attention_workspace_size(int C, int rows, int num_q_heads, const isd_kv_cache* kv, int max_len,
                                    int slices) {
  if (!kv || kv->num_kv_heads < 1 || (kv->head_dim != 64 && kv->head_dim != 128)) return 0;
  AttnPlan plan;
  if (plan_attention(C, rows, num_q_heads, kv, max_len, slices, &plan) != ISD_OK) return 0;
  return plan.total();
}

int isd_attention(const isd_kv_cache* kv, const void* q, const int32_t* ctx, int C, int rows, int num_q_heads,
                  float scale, int max_len, int slices, void* out, int odtype, void* ws, size_t ws_bytes,
                  int32_t* dev_err, hipStream_t stream) {
  return attention_call(kv, nullptr, nullptr, q, ctx, C, rows, num_q_heads, scale, max_len, slices, out, odtype, ws,
                        ws_bytes, dev_err, stream);
}

int isd_attention_with_block(const isd_kv_cache* kv, const void* k, const void* v, const void* q,
                             const int32_t* ctx, int C, int rows, int num_q_heads, float scale, int max_len, int slices,
                             void* out, int odtype, void* ws, size_t ws_bytes, int32_t* dev_err, hipStream_t stream) {
  if (!k || !v) return ISD_E_INVALID;
  if (!aligned16(k) || !aligned16(v)) return ISD_E_INVALID;
  return attention_call(kv, k, v, q, ctx, C, rows, num_q_heads, scale, max_len, slices, out, odtype, ws, ws_bytes,
                        dev_err, stream);
}

}  // extern "C"

namespace {

int attention_call(const isd_kv_cache* kv, const void* k_blk, const void* v_blk, const void* q, const int32_t* ctx,
                   int C, int rows, int num_q_heads, float scale, int max_len, int slices, void* out, int odtype,
                   void* ws, size_t ws_bytes, int32_t* dev_err, hipStream_t stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  if (odtype != ISD_F32 && odtype != ISD_BF16) return ISD_E_UNSUPPORTED;
  if (C == 0) return ISD_OK;
  if (!q || !ctx || !out) return ISD_E_INVALID;
  if (!(scale > 0.f) || !(scale < INFINITY)) return ISD_E_INVALID;
  if (!aligned16(q) || !aligned16(out)) return ISD_E_INVALID;
  AttnPlan plan;
  rc = plan_attention(C, rows, num_q_heads, kv, max_len, slices, &plan);
  if (rc) return rc;
  if (!ws || ws_bytes < plan.total() || !aligned16(ws)) return ISD_E_WORKSPACE;
  rc = isd_check_device_internal();
  if (rc) return rc;

  AttnParams p;
  p.k_pages = kv->k_pages;
  p.v_pages = kv->v_pages;
  p.block_table = kv->block_table;
  p.q = q;
  p.ctx = ctx;
  p.out = out;
  p.obf16 = odtype == ISD_BF16;
  char* w = static_cast<char*>(ws);
  p.tile_off = reinterpret_cast<int32_t*>(w);
  p.part_o = reinterpret_cast<float*>(w + plan.off_bytes);
  p.part_ml = reinterpret_cast<float*>(w + plan.off_bytes + plan.part_o_bytes);
  p.dev_err = dev_err;
  p.table_stride = kv->table_stride;
  p.num_pages = kv->num_pages;
  p.C = C;
  p.rows = rows;
  p.Hq = num_q_heads;
  p.Hkv = kv->num_kv_heads;
  p.group = num_q_heads / kv->num_kv_heads;
  p.M = p.group * rows;
  p.G = plan.G;
  p.MB = plan.MB;
  p.HPW = plan.HPW;
  p.CT = plan.CT;
  p.Kmax = plan.Kmax;
  int groups = plan.groups;
  if (plan.CT > 0) {
    // Few sequences and chunks (a single sequence, say) give fewer
    // workgroups than CUs. The heads per workgroup only group waves into
    // workgroups: a wave's arithmetic and the place of its partial in the
    // workspace do not depend on them. So they are halved until the grid
    // covers the CUs (the bound takes every sequence at max_len).
    const long cus = isd_device_cus_internal();
    while (p.HPW > 1 && static_cast<long>(p.Hkv / p.HPW) * p.G < cus) p.HPW /= 2;
    groups = p.Hkv / p.HPW;
  }
  p.scale_log2 = scale * kLog2e;
  p.k_blk = k_blk;
  p.v_blk = v_blk;

  hipError_t e;
  if (kv->dtype == ISD_BF16)
    e = kv->head_dim == 128 ? launch_attention_typed<uint16_t, 128>(p, groups, stream)
                            : launch_attention_typed<uint16_t, 64>(p, groups, stream);
  else
    e = kv->head_dim == 128 ? launch_attention_typed<float, 128>(p, groups, stream)
                            : launch_attention_typed<float, 64>(p, groups, stream);
  return e == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // namespace

extern "C" {

int isd_kv_write(const isd_kv_cache* kv, const void* k, const void* v, const int32_t* pos0, const int32_t* nrows,
                 int C, int rows, int32_t* dev_err, hipStream_t stream) {
  return kv_write_call(kv, 1, 0, k, v, pos0, nrows, C, rows, dev_err, stream);
}

int isd_kv_write_layers(const isd_kv_cache* kv, int layers, int64_t layer_stride, const void* k, const void* v,
                        const int32_t* pos0, const int32_t* nrows, int C, int rows, int32_t* dev_err,
                        hipStream_t stream) {
  if (layers < 0 || layer_stride < 0) return ISD_E_INVALID;
  if (layers > 65535) return ISD_E_UNSUPPORTED;  // layers map to a grid dimension
  if (layers > 1 && layer_stride < static_cast<int64_t>(kv ? kv->num_pages : 0) * (kv ? kv->num_kv_heads : 0) *
                                        (kv ? kv->head_dim : 0) * 16)
    return ISD_E_INVALID;  // the layers' pools would overlap
  if (layers == 0) return check_kv(kv);
  return kv_write_call(kv, layers, layer_stride, k, v, pos0, nrows, C, rows, dev_err, stream);
}

}  // extern "C"

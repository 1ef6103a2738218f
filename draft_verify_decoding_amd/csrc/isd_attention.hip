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
//  * Page layout (isd.h) makes every operand a run of 16 contiguous bytes:
//    K [Hkv][D/8][16 slots][8], V [Hkv][D][16 slots].
//  * Split-KV: a workgroup of 4 waves reduces one chunk of one (sequence,
//    KV head); waves interleave 32-key tiles and merge through LDS; units
//    with several chunks write (m, l, O) partials that a second kernel merges
//    in chunk order, so results do not depend on scheduling.
#include "isd_common.hpp"

namespace isd {

struct AttnParams {
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const void* q;
  const int32_t* ctx;
  float* out;
  float* part_o;   // [units][max_chunks][MB*32][D]
  float* part_ml;  // [units][max_chunks][MB*32][2]
  int32_t* dev_err;
  int table_stride, num_pages;
  int C, rows, Hq, Hkv, group, M;
  int chunk, max_chunks;
  float scale_log2;  // scale * log2(e)
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
  static __device__ __forceinline__ bf16x8 zero() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

  template <int D>
  static __device__ __forceinline__ void load_q(Regs<D>& r, const uint16_t* qrow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) r.q[s] = valid ? load16(qrow + 16 * s + 8 * hh) : zero();
  }
  // K operand: lane (row i, half hh) at k-step s holds dims 16s + 8hh .. +8
  // of tile key pi(i).
  template <int D>
  static __device__ __forceinline__ void load_k(Regs<D>& r, const uint16_t* kpage, bool valid, int slot, int hh) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      r.k[s] = valid ? load16(kpage + ((2 * s + hh) * 16 + slot) * 8) : zero();
  }
  // V^T operand: lane (dim d, half hh) at k-step p (= tile page p) holds
  // slots 8hh .. 8hh+7 of dim d. Keys at or past `limit` are zeroed.
  template <int D>
  static __device__ __forceinline__ void load_v(Regs<D>& r, const uint16_t* vpage, int p, bool valid, int lane32,
                                                int hh, int first_key, int limit) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      bf16x8 v = valid ? load16(vpage + (nb * 32 + lane32) * 16 + 8 * hh) : zero();
      if (first_key + 8 > limit) {
        u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (first_key + k >= limit) w[k >> 1] &= (k & 1) ? 0x0000ffffu : 0xffff0000u;
        v = __builtin_bit_cast(bf16x8, w);
      }
      r.v[nb][p] = v;
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
  template <int D>
  struct Regs {
    float q[D / 2];
    float k[D / 2];
    float v[D / 32][16];
  };
  template <int D>
  static __device__ __forceinline__ void load_q(Regs<D>& r, const float* qrow, bool valid, int hh) {
#pragma unroll
    for (int s = 0; s < D / 2; ++s) r.q[s] = valid ? qrow[2 * s + hh] : 0.f;
  }
  template <int D>
  static __device__ __forceinline__ void load_k(Regs<D>& r, const float* kpage, bool valid, int slot, int hh) {
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
      int d = 2 * s + hh;
      r.k[s] = valid ? kpage[((d >> 2) * 16 + slot) * 4 + (d & 3)] : 0.f;
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
        r.v[nb][8 * p + k] = ok ? vpage[(nb * 32 + lane32) * 16 + 8 * hh + k] : 0.f;
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

template <typename E, int D>
__device__ __forceinline__ const E* page_ptr(const void* pool, int pid, int Hkv, int g) {
  return static_cast<const E*>(pool) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16);
}

// One workgroup = 4 waves = one (chunk, sequence, KV head). Wave w handles
// query block rb = w % MB and interleaved tile stream ts = w / MB.
template <typename E, int D, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnParams p) {
  using Ops = AttnOps<E>;
  constexpr int SW = 4 / MB;  // tile streams per query block
  const int units = p.C * p.Hkv;
  const int unit = blockIdx.x % units;
  const int chunk = blockIdx.x / units;
  const int b = unit / p.Hkv;
  const int g = unit % p.Hkv;
  const int ctx = p.ctx[b];
  const int L = ctx + p.rows;  // positions 0 .. L-1 are read
  const int c0 = chunk * p.chunk;
  if (ctx < 0) {
    if (chunk == 0 && threadIdx.x == 0) set_dev_err(p.dev_err, ISD_DEV_STATE);
    return;
  }
  const int nchunks = (L + p.chunk - 1) / p.chunk;
  if (nchunks > p.max_chunks) {  // ctx + rows exceeds the max_len the grid was sized for
    if (chunk == 0 && threadIdx.x == 0) set_dev_err(p.dev_err, ISD_DEV_CAPACITY);
    return;
  }
  if (c0 >= L) return;
  const int c1 = min(L, c0 + p.chunk);

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int lane32 = lane & 31;
  const int hh = lane >> 5;
  const int rb = wave % MB;
  const int ts = wave / MB;

  // Query column of this lane.
  const int qi = rb * 32 + lane32;
  const bool qvalid = qi < p.M;
  const int hl = qvalid ? qi / p.rows : 0;
  const int irow = qvalid ? qi % p.rows : p.rows - 1;
  const int h = g * p.group + hl;
  const int vis_limit = ctx + irow;  // last visible position

  typename Ops::template Regs<D> r;
  const E* qrow = static_cast<const E*>(p.q) + ((static_cast<size_t>(b) * p.rows + irow) * p.Hq + h) * D;
  Ops::template load_q<D>(r, qrow, qvalid, hh);

  f32x16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = f32x16{};
  float m_run = -1e30f;  // finite floor: exp2(m_old - m_new) stays defined
  float l_run = 0.f;

  const int32_t* table = p.block_table + static_cast<size_t>(b) * p.table_stride;
  const int krow_key = tile_key_of_row(lane32);  // tile key this lane loads for K
  uint32_t err = 0;

  for (int t0 = c0 + 32 * ts; t0 < c1; t0 += 32 * SW) {
    // Resolve the tile's two pages.
    const E* kp[2];
    const E* vp[2];
    bool pv_ok[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int first = t0 + 16 * pg;
      bool ok = first < L;
      int pid = 0;
      if (ok) {
        const int col = first >> 4;
        if (col >= p.table_stride) {
          err |= ISD_DEV_CAPACITY;
          ok = false;
        } else {
          pid = table[col];
          if (pid < 0 || pid >= p.num_pages) {
            err |= ISD_DEV_PAGE_OOB;
            ok = false;
          }
        }
      }
      pv_ok[pg] = ok;
      kp[pg] = page_ptr<E, D>(p.k_pages, ok ? pid : 0, p.Hkv, g);
      vp[pg] = page_ptr<E, D>(p.v_pages, ok ? pid : 0, p.Hkv, g);
    }
    {
      const int kpg = krow_key >> 4;
      Ops::template load_k<D>(r, kpg ? kp[1] : kp[0], pv_ok[kpg], krow_key & 15, hh);
    }
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
      Ops::template load_v<D>(r, vp[pg], pg, pv_ok[pg], lane32, hh, t0 + 16 * pg + 8 * hh, L);

    f32x16 s = Ops::template qk<D>(r);

    float sv[16];
    float tmax = -INFINITY;
    const bool need_mask = t0 + 31 > ctx;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = s[e];
      if (need_mask) {
        const int key = t0 + tile_key_of_reg(e, hh);
        x = (key <= vis_limit) ? x : -INFINITY;
      }
      sv[e] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax * p.scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float pr[16];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pr[e] = fast_exp2(fmaf(sv[e], p.scale_log2, -m_new));
      psum += pr[e];
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb][e] *= alpha;
    Ops::template pv<D>(r, pr, o);
  }
  if (err) set_dev_err(p.dev_err, err);

  // Lane-half partial sums -> per-column totals.
  l_run += shfl_xor_f(l_run, 32);

  // Merge the SW tile streams of each query block through LDS.
  __shared__ float s_o[4][D][33];
  __shared__ float s_m[4][32];
  __shared__ float s_l[4][32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = nb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
      s_o[wave][d][lane32] = o[nb][e];
    }
  if (hh == 0) {
    s_m[wave][lane32] = m_run;
    s_l[wave][lane32] = l_run;
  }
  __syncthreads();

  const bool final_out = nchunks == 1;
  for (int idx = threadIdx.x; idx < MB * 32 * D; idx += 256) {
    const int d = idx % D;
    const int j = (idx / D) % 32;
    const int qb = idx / (32 * D);
    const int col = qb * 32 + j;
    if (col >= p.M) continue;
    float mstar = -1e30f;
#pragma unroll
    for (int st = 0; st < SW; ++st) mstar = fmaxf(mstar, s_m[qb + MB * st][j]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int st = 0; st < SW; ++st) {
      const int w = qb + MB * st;
      const float wt = fast_exp2(s_m[w][j] - mstar);
      acc = fmaf(wt, s_o[w][d][j], acc);
      lsum = fmaf(wt, s_l[w][j], lsum);
    }
    if (final_out) {
      const int hl2 = col / p.rows, i2 = col % p.rows;
      const int h2 = g * p.group + hl2;
      p.out[((static_cast<size_t>(b) * p.rows + i2) * p.Hq + h2) * D + d] = acc / lsum;
    } else {
      const size_t base = (static_cast<size_t>(unit) * p.max_chunks + chunk) * (MB * 32) + col;
      p.part_o[base * D + d] = acc;
      if (d == 0) {
        p.part_ml[base * 2] = mstar;
        p.part_ml[base * 2 + 1] = lsum;
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, KV head) in
// chunk order. One workgroup per unit and query block.
template <int D, int MB>
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnParams p) {
  const int unit = blockIdx.x;
  const int qb = blockIdx.y;
  const int b = unit / p.Hkv;
  const int g = unit % p.Hkv;
  const int ctx = p.ctx[b];
  if (ctx < 0) return;
  const int L = ctx + p.rows;
  const int nchunks = (L + p.chunk - 1) / p.chunk;
  if (nchunks <= 1 || nchunks > p.max_chunks) return;
  for (int idx = threadIdx.x; idx < 32 * D; idx += 256) {
    const int d = idx % D;
    const int col = qb * 32 + idx / D;
    if (col >= p.M) continue;
    const size_t base0 = static_cast<size_t>(unit) * p.max_chunks * (MB * 32) + col;
    float mstar = -1e30f;
    for (int c = 0; c < nchunks; ++c) mstar = fmaxf(mstar, p.part_ml[(base0 + c * (MB * 32)) * 2]);
    float acc = 0.f, lsum = 0.f;
    for (int c = 0; c < nchunks; ++c) {
      const size_t base = base0 + static_cast<size_t>(c) * (MB * 32);
      const float wt = fast_exp2(p.part_ml[base * 2] - mstar);
      acc = fmaf(wt, p.part_o[base * D + d], acc);
      lsum = fmaf(wt, p.part_ml[base * 2 + 1], lsum);
    }
    const int hl = col / p.rows, i = col % p.rows;
    const int h = g * p.group + hl;
    p.out[((static_cast<size_t>(b) * p.rows + i) * p.Hq + h) * D + d] = acc / lsum;
  }
}

// ----------------------------------------------------------------- KV write
template <typename E, int D>
__global__ __launch_bounds__(256) void kv_write_kernel(void* k_pages, void* v_pages, const int32_t* block_table,
                                                       int table_stride, int num_pages, int Hkv, const E* k,
                                                       const E* v, const int32_t* pos0, const int32_t* nrows, int C,
                                                       int rows, int32_t* dev_err) {
  constexpr int KP = Elem<E>::kPerVec;
  const int per_row = Hkv * (D / KP);
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(C) * rows * per_row) return;
  const int c = static_cast<int>(idx % (D / KP));
  const int g = static_cast<int>((idx / (D / KP)) % Hkv);
  const int r = static_cast<int>((idx / per_row) % rows);
  const int b = static_cast<int>(idx / (static_cast<long>(per_row) * rows));
  const int nr = nrows ? nrows[b] : rows;
  if (r >= nr) return;
  const int pos = pos0[b] + r;
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
  const size_t src = ((static_cast<size_t>(b) * rows + r) * Hkv + g) * D + c * KP;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
  E* kpage = static_cast<E*>(k_pages) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16);
  E* vpage = static_cast<E*>(v_pages) + (static_cast<size_t>(pid) * Hkv + g) * (D * 16);
  *reinterpret_cast<u32x4*>(kpage + (c * 16 + slot) * KP) = kv;
  const E* ve = reinterpret_cast<const E*>(&vv);
#pragma unroll
  for (int j = 0; j < KP; ++j) vpage[(c * KP + j) * 16 + slot] = ve[j];
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

int auto_chunk(int units, int max_len) {
  // Aim at about 1024 workgroups of 4 waves, tiles of 32 keys.
  long want = (static_cast<long>(units) * max_len + 1023) / 1024;
  long c = ((want + 31) / 32) * 32;
  if (c < 64) c = 64;
  if (c > 4096) c = 4096;
  return static_cast<int>(c);
}

struct AttnPlan {
  int chunk, max_chunks, MB;
  size_t part_o_bytes, part_ml_bytes;
};

int plan_attention(int C, int rows, int Hq, const isd_kv_cache* kv, int max_len, int chunk, AttnPlan* plan) {
  if (C < 0 || rows < 1 || rows > 64 || Hq < 1) return ISD_E_INVALID;
  const int Hkv = kv->num_kv_heads;
  if (Hq % Hkv != 0) return ISD_E_UNSUPPORTED;
  const int M = (Hq / Hkv) * rows;
  if (M > 128) return ISD_E_UNSUPPORTED;
  if (max_len < rows) return ISD_E_INVALID;
  if (chunk < 0 || chunk % 32 != 0) return ISD_E_INVALID;
  plan->MB = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  plan->chunk = chunk ? chunk : auto_chunk(C * Hkv, max_len);
  plan->max_chunks = (max_len + plan->chunk - 1) / plan->chunk;
  const size_t cols = static_cast<size_t>(C) * Hkv * plan->max_chunks * plan->MB * 32;
  if (plan->max_chunks > 1) {
    plan->part_o_bytes = cols * kv->head_dim * sizeof(float);
    plan->part_ml_bytes = cols * 2 * sizeof(float);
  } else {
    plan->part_o_bytes = plan->part_ml_bytes = 0;
  }
  return ISD_OK;
}

template <typename E, int D>
hipError_t launch_attention_typed(const AttnParams& p, int MB, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.C * p.Hkv * p.max_chunks));
  const dim3 mgrid(static_cast<unsigned>(p.C * p.Hkv), static_cast<unsigned>(MB));
  switch (MB) {
    case 1:
      hipLaunchKernelGGL((attention_kernel<E, D, 1>), grid, dim3(256), 0, stream, p);
      if (p.max_chunks > 1) hipLaunchKernelGGL((attention_merge_kernel<D, 1>), mgrid, dim3(256), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((attention_kernel<E, D, 2>), grid, dim3(256), 0, stream, p);
      if (p.max_chunks > 1) hipLaunchKernelGGL((attention_merge_kernel<D, 2>), mgrid, dim3(256), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((attention_kernel<E, D, 4>), grid, dim3(256), 0, stream, p);
      if (p.max_chunks > 1) hipLaunchKernelGGL((attention_merge_kernel<D, 4>), mgrid, dim3(256), 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

size_t isd_attention_workspace_size(int C, int rows, int num_q_heads, const isd_kv_cache* kv, int max_len,
                                    int chunk) {
  if (!kv || kv->num_kv_heads < 1 || (kv->head_dim != 64 && kv->head_dim != 128)) return 0;
  AttnPlan plan;
  if (plan_attention(C, rows, num_q_heads, kv, max_len, chunk, &plan) != ISD_OK) return 0;
  return plan.part_o_bytes + plan.part_ml_bytes;
}

int isd_attention(const isd_kv_cache* kv, const void* q, const int32_t* ctx, int C, int rows, int num_q_heads,
                  float scale, int max_len, int chunk, float* out, void* ws, size_t ws_bytes, int32_t* dev_err,
                  hipStream_t stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  if (C == 0) return ISD_OK;
  if (!q || !ctx || !out) return ISD_E_INVALID;
  if (!(scale > 0.f) || !(scale < INFINITY)) return ISD_E_INVALID;
  if (!aligned16(q) || !aligned16(out)) return ISD_E_INVALID;
  AttnPlan plan;
  rc = plan_attention(C, rows, num_q_heads, kv, max_len, chunk, &plan);
  if (rc) return rc;
  const size_t need = plan.part_o_bytes + plan.part_ml_bytes;
  if (need && (!ws || ws_bytes < need || !aligned16(ws))) return ISD_E_WORKSPACE;
  rc = isd_check_device_internal();
  if (rc) return rc;

  AttnParams p;
  p.k_pages = kv->k_pages;
  p.v_pages = kv->v_pages;
  p.block_table = kv->block_table;
  p.q = q;
  p.ctx = ctx;
  p.out = out;
  p.part_o = need ? static_cast<float*>(ws) : nullptr;
  p.part_ml = need ? reinterpret_cast<float*>(static_cast<char*>(ws) + plan.part_o_bytes) : nullptr;
  p.dev_err = dev_err;
  p.table_stride = kv->table_stride;
  p.num_pages = kv->num_pages;
  p.C = C;
  p.rows = rows;
  p.Hq = num_q_heads;
  p.Hkv = kv->num_kv_heads;
  p.group = num_q_heads / kv->num_kv_heads;
  p.M = p.group * rows;
  p.chunk = plan.chunk;
  p.max_chunks = plan.max_chunks;
  p.scale_log2 = scale * kLog2e;

  hipError_t e;
  if (kv->dtype == ISD_BF16)
    e = kv->head_dim == 128 ? launch_attention_typed<uint16_t, 128>(p, plan.MB, stream)
                            : launch_attention_typed<uint16_t, 64>(p, plan.MB, stream);
  else
    e = kv->head_dim == 128 ? launch_attention_typed<float, 128>(p, plan.MB, stream)
                            : launch_attention_typed<float, 64>(p, plan.MB, stream);
  return e == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

int isd_kv_write(const isd_kv_cache* kv, const void* k, const void* v, const int32_t* pos0, const int32_t* nrows,
                 int C, int rows, int32_t* dev_err, hipStream_t stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  if (C < 0 || rows < 0) return ISD_E_INVALID;
  if (C == 0 || rows == 0) return ISD_OK;
  if (!k || !v || !pos0) return ISD_E_INVALID;
  if (!aligned16(k) || !aligned16(v)) return ISD_E_INVALID;
  rc = isd_check_device_internal();
  if (rc) return rc;
  const int D = kv->head_dim;
  const int KP = kv->dtype == ISD_BF16 ? 8 : 4;
  const long total = static_cast<long>(C) * rows * kv->num_kv_heads * (D / KP);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
#define ISD_KVW(E, DD)                                                                                          \
  hipLaunchKernelGGL((kv_write_kernel<E, DD>), grid, dim3(256), 0, stream, kv->k_pages, kv->v_pages,            \
                     kv->block_table, kv->table_stride, kv->num_pages, kv->num_kv_heads, static_cast<const E*>(k), \
                     static_cast<const E*>(v), pos0, nrows, C, rows, dev_err)
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

}  // extern "C"

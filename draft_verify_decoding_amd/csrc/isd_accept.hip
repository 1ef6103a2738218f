// The accept side of one ISD step on gfx950: vocab softmax statistics, the
// min(1, p/q) test, the residual or bonus draw and the next drafts.
//
// What the step computes is fixed by the I-DLM page (fr.news.hada.io,
// "Documentation et ressources > Inference & ISD": proposals q at MASK
// positions, verification p at clean positions, keep a draft with
// probability min(1, p(x)/q(x)), which keeps the AR distribution). The
// residual draw normalize(max(0, p - q)) after the first rejection is the
// standard rejection-sampling step behind that guarantee; the bonus draw and
// the FULL/FRESH alternation are what reproduce the page's tokens-per-forward
// closed form ("Speedup Factor Explorer").
//
// Two launches:
//   stats   one workgroup per 8192-entry chunk of every logits row the step
//           reads: the chunk's max and sum of exp(l - max) (fp32 from exact
//           bf16), streamed with non-temporal loads; the workgroup whose
//           chunk holds a pending draft also records that draft's logit in
//           its verify row. Nothing else: the launch is a pure stream.
//   decide  grid (slices, sequences). Every workgroup of a sequence merges
//           the chunk statistics into row statistics and takes the accept
//           decision (same fixed-order arithmetic, so all agree); slice 0
//           writes the outputs the decision alone fixes. Then:
//           - all drafts pass: slice k draws row n + k (the bonus for k = 0,
//             proposal k after) from one rescanned chunk and writes it;
//           - a draft is rejected: slice k sums max(0, P_a - Q_{a+1}) over
//             one chunk; the last slice of the sequence to count itself in
//             (a counter per sequence, cleared by the stats launch) picks
//             the chunk of the residual draw, rescans it and writes the
//             token. Slice sums go through agent-scope atomic stores and
//             loads; a writer waits for its stores to complete before it
//             counts itself in.
// When the caller passes the chunk statistics (isd_lm_head wrote them with
// the logits), a small launch that clears the counters and gathers the
// drafts' logits replaces the stats launch.
#include <mutex>

#include "isd_common.hpp"

namespace isd {

constexpr int kChunk = kVocabChunk;  // vocab entries per stats chunk
constexpr int kThreads = 256;        // threads per workgroup
constexpr int kPerThread = 32;       // entries per thread in a chunk
constexpr int kResidChunks = 1;      // chunks per residual slice
constexpr int kMaxN = 8;
constexpr int kMaxChunks = 64;  // vocabularies up to 524,288 entries
static_assert(kThreads * kPerThread == kChunk, "chunk tiling");

struct AcceptParams {
  const void* logits;
  const void* prev_logits;
  long ld;
  int C, N, V, rows, nch, ns;
  isd_seq_state in, out;
  uint64_t seed, step;
  const uint64_t* step_dev;  // when set, the step number comes from here
  int32_t *accepted, *n_emit, *emit, *kv_commit, *ctx;
  float *p_x, *resid_mass, *row_m, *row_s;
  float2* stats;  // [C][rows][nch] (chunk max, chunk sum), or the given ones
  float* lx;      // [C][kMaxN] logit of draft j+1 in verify row j
  float* resid;   // [C][nch] residual sum per chunk
  int* arrive;    // [C] workgroups of the decide launch done, per sequence
  int32_t* dev_err;
  int argmax;  // proposals are argmax q (a point mass at the draft)
};

// --------------------------------------- values handed between workgroups
// The residual slices hand their sums to the last slice of their sequence.
// Each value goes through a device-coherent (agent-scope) store and load,
// which reach the coherence point of the 8 XCDs directly. The writer waits
// until its stores are complete (stores_done: s_waitcnt 0, with compiler
// barriers on both sides) before its relaxed add on the sequence's counter,
// and the reader issues its loads only after that add has returned the
// count that makes it last, so no load can see a value older than the
// store. Release/acquire ordering on the add would also order the stores,
// but at agent scope gfx950 implements it as a writeback (release) and an
// invalidation (acquire) of the XCD's L2: a probe of 2,240 counted tasks
// took 34 us that way against 5 us with relaxed adds.
__device__ __forceinline__ void stores_done() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void put_f32(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_f32(float* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ Philox4x64-10
// Salmon et al., SC'11: two 64x64->128 multiplies per round, Weyl key bumps,
// ten rounds. Counter (slot, b, step, 0), key (seed, 0).
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                 uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}
__device__ __forceinline__ float uniform_of(uint64_t w0) {
  return (static_cast<float>(static_cast<uint32_t>(w0 >> 41)) + 0.5f) * 0x1p-23f;
}
__device__ __forceinline__ float slot_uniform(const AcceptParams& p, int slot, int b) {
  const uint64_t step = p.step_dev ? *p.step_dev : p.step;
  return uniform_of(philox_word0(static_cast<uint64_t>(slot), static_cast<uint64_t>(b), step, 0ull, p.seed, 0ull));
}

// -------------------------------------------------------------- arithmetic
// weight_of, prob_of and merge_ms (isd_common.hpp) are the only places that
// turn logits into softmax weights, so equal inputs give equal bits.

template <typename E>
__device__ __forceinline__ const E* row_ptr(const void* base, long ld, int rows, int b, int r) {
  return static_cast<const E*>(base) + (static_cast<long>(b) * rows + r) * ld;
}

template <typename E>
__device__ __forceinline__ float load_elem(const E* row, int v) {
  return Elem<E>::to_f32(row[v]);
}

// This thread's 32 entries of a chunk, kept packed as loaded (bf16 pairs
// or fp32 words); at(k) unpacks entry k exactly. Keeping the rows packed
// and recomputing weights where they are needed holds the register
// footprint of the rescans down.
template <typename E>
struct Raw;
template <>
struct Raw<uint16_t> {
  static constexpr uint32_t kNegInf = 0xff80ff80u;  // two bf16 -inf
  u32x4 v[kPerThread / 8];
  __device__ __forceinline__ float at(int k) const {
    const uint32_t w = v[k >> 3][(k >> 1) & 3];
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  // opaque to the optimiser: values recomputed after this are not reused
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int q = 0; q < kPerThread / 8; ++q) asm volatile("" : "+v"(v[q]));
  }
};
template <>
struct Raw<float> {
  u32x4 v[kPerThread / 4];
  __device__ __forceinline__ float at(int k) const { return __uint_as_float(v[k >> 2][k & 3]); }
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q) asm volatile("" : "+v"(v[q]));
  }
};

// 16 bytes of entries v0 .. v0 + KP - 1 of a row; entries >= V read as -inf.
// NT: a streaming (non-temporal) load, for data read once.
template <bool NT = false>
__device__ __forceinline__ u32x4 load_vec(const uint16_t* row, int V, int v0) {
  if (v0 + 8 <= V) {
    const u32x4* ptr = reinterpret_cast<const u32x4*>(row + v0);
    return NT ? __builtin_nontemporal_load(ptr) : *ptr;
  }
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = v0 + 2 * i < V ? row[v0 + 2 * i] : 0xff80u;
    const uint32_t hi = v0 + 2 * i + 1 < V ? row[v0 + 2 * i + 1] : 0xff80u;
    w[i] = lo | (hi << 16);
  }
  return w;
}
template <bool NT = false>
__device__ __forceinline__ u32x4 load_vec(const float* row, int V, int v0) {
  if (v0 + 4 <= V) {
    const u32x4* ptr = reinterpret_cast<const u32x4*>(row + v0);
    return NT ? __builtin_nontemporal_load(ptr) : *ptr;
  }
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = v0 + i < V ? __float_as_uint(row[v0 + i]) : __float_as_uint(-INFINITY);
  return w;
}

// Entries c*kChunk + 32t .. +31 of chunk c go to thread t (token order
// within a thread, as the inverse-CDF search needs).
template <typename E>
__device__ __forceinline__ Raw<E> load_slice(const E* row, int V, int c) {
  constexpr int KP = Elem<E>::kPerVec;
  Raw<E> r;
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
#pragma unroll
  for (int q = 0; q < kPerThread / KP; ++q) r.v[q] = load_vec(row, V, v0 + q * KP);
  return r;
}

// Entries c*kChunk + i*kThreads*KP + KP*t .. +KP-1 of chunk c go to thread
// t: each load instruction of the workgroup reads 4 KB of contiguous logits.
// (A chunk's max and sum do not depend on which thread holds what.) The
// statistics pass reads every row once: streaming loads, which measured
// twice as fast as cached ones on a cold 130 MB batch of rows.
template <typename E>
__device__ __forceinline__ Raw<E> load_coalesced(const E* row, int V, int c) {
  constexpr int KP = Elem<E>::kPerVec;
  Raw<E> r;
#pragma unroll
  for (int q = 0; q < kPerThread / KP; ++q)
    r.v[q] = load_vec<true>(row, V, c * kChunk + q * kThreads * KP + threadIdx.x * KP);
  return r;
}

// Workgroup reduction of (max, sum) pairs in a fixed tree.
__device__ __forceinline__ void block_reduce_ms(float& m, float& s) {
  __shared__ float sm[kThreads / kWave], ss[kThreads / kWave];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) merge_ms(m, s, __shfl_xor(m, off, kWave), __shfl_xor(s, off, kWave));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    sm[w] = m;
    ss[w] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) merge_ms(m, s, sm[i], ss[i]);
  __syncthreads();
}

__device__ __forceinline__ float block_sum(float v) {
  __shared__ float sv[kThreads / kWave];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  if ((threadIdx.x % kWave) == 0) sv[threadIdx.x / kWave] = v;
  __syncthreads();
  float t = sv[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) t += sv[i];
  __syncthreads();
  return t;
}

// Exclusive prefix over threads (thread order) of v; returns the prefix.
__device__ __forceinline__ float block_exclusive_scan(float v) {
  __shared__ float sw[kThreads / kWave];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  float inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  float excl = __shfl_up(inc, 1, kWave);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) sw[w] = inc;
  __syncthreads();
  float base = 0.f;
  for (int i = 0; i < w; ++i) base += sw[i];
  __syncthreads();
  return base + excl;
}

// (max, sum) of a row from its chunk statistics, merged in chunk order.
__device__ __forceinline__ float2 row_ms(const float2* st, int nch) {
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, st[c].x);
  float S = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < nch; ++c) S += st[c].y * fast_exp2((st[c].x - M) * kLog2e);
  }
  return make_float2(M, S);
}
__device__ __forceinline__ bool ms_finite(float2 ms) {
  return ms.x > -INFINITY && ms.x < INFINITY && ms.y > 0.f && ms.y < INFINITY;
}

// Residual weight max(0, P_a(v) - Q(v)) of one entry.
// Both products are rounded before the subtraction (no fused multiply-add),
// so equal P and Q cancel exactly.
__device__ __forceinline__ float resid_weight(float l, float lq, float ma_l2, float inv_sa, float mq_l2, float inv_sq) {
#pragma clang fp contract(off)
  const float pa = weight_of(l, ma_l2) * inv_sa;
  const float qa = weight_of(lq, mq_l2) * inv_sq;
  return fmaxf(0.f, pa - qa);
}

// Inverse-CDF search inside one chunk: wf(k) is this thread's weight of
// entry c*kChunk + 32t + k (thread order = token order), the target t_rel
// is measured from the start of the chunk. Returns the smallest crossing
// token id, or the last token with non-zero weight in the chunk when
// rounding leaves no crossing; *w_tok is that token's weight. The thread
// that holds the crossing recomputes its weights in the same order (after
// fence()) rather than keeping all 32 of them live across the scan.
template <typename WF>
__device__ __forceinline__ int chunk_search(WF& wf, int c, float t_rel, float* w_tok) {
  __shared__ int s_tok, s_last;
  __shared__ float s_wtok, s_wlast;
  if (threadIdx.x == 0) {
    s_tok = 0x7fffffff;
    s_last = -1;
  }
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
  float local = 0.f, w_last = 0.f;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const float w = wf(k);
    local += w;
    if (w > 0.f) {
      last = v0 + k;
      w_last = w;
    }
  }
  const float base = block_exclusive_scan(local);  // also syncs
  const float tr = t_rel - base;
  wf.fence();
  int hit = -1;
  float w_hit = 0.f;
  if (tr >= 0.f && local > tr) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float w = wf(k);
      acc += w;
      if (hit < 0 && acc > tr) {
        hit = v0 + k;
        w_hit = w;
      }
    }
    if (hit >= 0) atomicMin(&s_tok, hit);
  }
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (hit >= 0 && hit == s_tok) s_wtok = w_hit;
  if (last >= 0 && last == s_last) s_wlast = w_last;
  __syncthreads();
  const bool crossed = s_tok != 0x7fffffff;
  const int tok = crossed ? s_tok : s_last;
  *w_tok = crossed ? s_wtok : s_wlast;
  __syncthreads();
  return tok;
}

// Softmax weight of a row's entries relative to its max (log2 units).
template <typename E>
struct SoftmaxWeights {
  Raw<E> x;
  float ml;
  __device__ __forceinline__ float operator()(int k) const { return weight_of(x.at(k), ml); }
  __device__ __forceinline__ void fence() { x.fence(); }
};

// Choose the chunk of a row whose (rescaled) chunk sums cross t.
// Returns the chunk and writes the target relative to its start.
__device__ __forceinline__ int pick_chunk_from_stats(const float2* st, int nch, float M, float t, float* t_rel) {
  float run = 0.f;
  int last_nz = 0;
  for (int c = 0; c < nch; ++c) {
    const float wc = st[c].y * fast_exp2((st[c].x - M) * kLog2e);
    if (wc > 0.f) last_nz = c;
    if (run + wc > t) {
      *t_rel = t - run;
      return c;
    }
    run += wc;
  }
  *t_rel = INFINITY;  // rounding: take the last non-zero token of that chunk
  return last_nz;
}

// Sample from softmax(row r) (max M, sum S, chunk statistics st in LDS)
// with uniform u: returns the token (every thread) and its probability.
template <typename E>
__device__ __forceinline__ int sample_row(const AcceptParams& p, int b, int r, const float2* st, float M, float S,
                                          float u, float* prob) {
  __shared__ int s_c;
  __shared__ float s_trel;
  if (threadIdx.x == 0) {
    float t_rel;
    s_c = pick_chunk_from_stats(st, p.nch, M, u * S, &t_rel);
    s_trel = t_rel;
  }
  __syncthreads();
  const int c = s_c;
  const float t_rel = s_trel;
  SoftmaxWeights<E> wf{load_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, r), p.V, c), M * kLog2e};
  float w;
  const int tok = chunk_search(wf, c, t_rel, &w);
  *prob = w / S;  // = prob_of(l(tok), M, S): the same weight, divided by S
  return tok;
}

// argmax of row r, ties to the smallest id: the first chunk whose maximum is
// the row maximum holds it; its entries are compared exactly with that value.
template <typename E>
__device__ __forceinline__ int argmax_row(const AcceptParams& p, int b, int r, const float2* st, float M) {
  __shared__ int s_tok;
  int c = 0;
  while (c + 1 < p.nch && st[c].x != M) ++c;
  if (threadIdx.x == 0) s_tok = 0x7fffffff;
  __syncthreads();
  const Raw<E> x = load_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, r), p.V, c);
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
  int hit = 0x7fffffff;
#pragma unroll
  for (int k = kPerThread - 1; k >= 0; --k)
    if (x.at(k) == M) hit = v0 + k;
  if (hit != 0x7fffffff) atomicMin(&s_tok, hit);
  __syncthreads();
  const int tok = s_tok;
  __syncthreads();
  return tok;
}

// What the residual of a sequence that rejected draft a+1 needs.
struct ResidArgs {
  float Ma, Sa;  // row a's statistics
  float qm, qs;  // statistics of the q row that proposed draft a+1
  int a, qrow, x_rej;
};

// Residual weights max(0, P_a - Q_{a+1}) of this thread's slice of chunk
// c. With argmax proposals Q_{a+1} is a point mass at the rejected draft:
// the residual is P_a with that token removed, and the previous block is
// not read.
template <typename E>
struct ResidWeights {
  Raw<E> x, y;
  float ma_l2, inv_sa, mq_l2, inv_sq;
  int v0, x_rej, argmax;
  __device__ __forceinline__ float operator()(int k) const {
    const float l = x.at(k);
    if (argmax) {
#pragma clang fp contract(off)
      const float pa = weight_of(l, ma_l2) * inv_sa;
      return (l == -INFINITY || v0 + k == x_rej) ? 0.f : pa;
    }
    return l == -INFINITY ? 0.f : resid_weight(l, y.at(k), ma_l2, inv_sa, mq_l2, inv_sq);
  }
  __device__ __forceinline__ void fence() {
    x.fence();
    y.fence();
  }
};

template <typename E>
__device__ __forceinline__ ResidWeights<E> resid_weights(const AcceptParams& p, int b, const ResidArgs& ra, int c) {
  ResidWeights<E> r;
  r.x = load_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, ra.a), p.V, c);
  if (!p.argmax) r.y = load_slice<E>(row_ptr<E>(p.prev_logits, p.ld, p.rows, b, ra.qrow + ra.a), p.V, c);
  r.ma_l2 = ra.Ma * kLog2e;
  r.inv_sa = 1.f / ra.Sa;
  r.mq_l2 = ra.qm * kLog2e;
  r.inv_sq = 1.f / ra.qs;
  r.v0 = c * kChunk + threadIdx.x * kPerThread;
  r.x_rej = ra.x_rej;
  r.argmax = p.argmax;
  return r;
}

// Pending drafts of sequence b (an invalid count reads as 0; the decide
// launch flags it).
__device__ __forceinline__ int seq_n(const AcceptParams& p, int b) {
  const int n = p.in.n_draft[b];
  return (n < 0 || n > p.N - 1) ? 0 : n;
}

// ============================================================ stats kernel
// Grid (chunks, 2N-1 rows, sequences): chunk c of row r of sequence b, if
// the step reads that row (rows 0 .. n+N-1).
template <typename E>
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(AcceptParams p) {
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  if (c == 0 && r == 0 && threadIdx.x == 0) p.arrive[b] = 0;  // the decide launch counts from zero
  const int n = seq_n(p, b);
  if (r > n + p.N - 1) return;
  const Raw<E> x = load_coalesced<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, r), p.V, c);
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) m = fmaxf(m, x.at(k));
  float s = 0.f;
  if (m != -INFINITY) {
    const float ml = m * kLog2e;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) s += weight_of(x.at(k), ml);
  }
  // the logit of draft r+1 in verify row r, by the thread that holds it
  if (r < n) {
    constexpr int KP = Elem<E>::kPerVec;
    const int o = p.in.drafts[b * (p.N - 1) + r] - c * kChunk;
    if (o >= 0 && o < kChunk && o + c * kChunk < p.V && (o % (kThreads * KP)) / KP == static_cast<int>(threadIdx.x)) {
      const int kk = (o / (kThreads * KP)) * KP + o % KP;
      float l = 0.f;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (k == kk) l = x.at(k);
      p.lx[b * kMaxN + r] = l;
    }
  }
  block_reduce_ms(m, s);
  if (threadIdx.x == 0) p.stats[(static_cast<long>(b) * p.rows + r) * p.nch + c] = make_float2(m, s);
}

// With the chunk statistics given: clear the counters and gather the
// drafts' logits. One thread per (sequence, verify row).
template <typename E>
__global__ __launch_bounds__(256) void accept_prep_kernel(AcceptParams p) {
  const int nd = p.N - 1;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.C * nd) return;
  const int b = i / nd, j = i % nd;
  if (j == 0) p.arrive[b] = 0;
  const int d = p.in.drafts[b * nd + j];
  if (j < seq_n(p, b) && d >= 0 && d < p.V) p.lx[b * kMaxN + j] = load_elem(row_ptr<E>(p.logits, p.ld, p.rows, b, j), d);
}

// ------------------------------------------------ per-sequence decision
// Row statistics, uniforms and the accept decision of sequence b; every
// workgroup of the decide launch computes the same values.
struct Decision {
  int n, a, err, qrow;
  float2 ms[2 * kMaxN];                // row (max, sum)
  float u[2 * kMaxN];                  // uniforms by slot
  float px[kMaxN];                     // P_{j-1}(x_j) of tested drafts, NaN otherwise
  float2 st[2 * kMaxN - 1][kMaxChunks];  // chunk statistics of the rows read
};

template <typename E>
__device__ __forceinline__ void decide(const AcceptParams& p, int b, Decision& d) {
  const int tid = threadIdx.x, N = p.N, nd = N - 1, R = 2 * N - 1, nch = p.nch;
  __shared__ int s_nraw, s_draft[kMaxN];
  __shared__ float s_qx[kMaxN], s_lx[kMaxN];
  // everything in one round trip: the statistics of every row the step may
  // read (those past n+N-1 are not used), the state, the drafts' logits
  for (int i = tid; i < R * nch; i += kThreads)
    d.st[i / nch][i % nch] = p.stats[(static_cast<long>(b) * p.rows + i / nch) * nch + i % nch];
  if (tid == kThreads - 1) {
    s_nraw = p.in.n_draft[b];
    d.qrow = p.in.q_row[b];
  }
  if (tid >= kThreads - 1 - kMaxN && tid < kThreads - 1 - kMaxN + nd) {
    const int j = tid - (kThreads - 1 - kMaxN);
    s_draft[j] = p.in.drafts[b * nd + j];
    s_qx[j] = p.in.q_x[b * nd + j];
    s_lx[j] = p.lx[b * kMaxN + j];
  }
  if (tid < 2 * N) d.u[tid] = slot_uniform(p, tid, b);
  __syncthreads();
  const int n_raw = s_nraw;
  const int n = (n_raw < 0 || n_raw > nd) ? 0 : n_raw;
  if (tid < n + N) d.ms[tid] = row_ms(d.st[tid], nch);
  __syncthreads();
  if (tid == 0) {
    int err = 0;
    if (n_raw < 0 || n_raw > nd) err |= ISD_DEV_STATE;
    if (n > 0 && ((!p.argmax && !p.prev_logits) || d.qrow < 0 || d.qrow + n - 1 >= p.rows)) err |= ISD_DEV_STATE;
    for (int j = 0; j < n; ++j)
      if (s_draft[j] < 0 || s_draft[j] >= p.V) err |= ISD_DEV_TOKEN_OOB;
    for (int r = 0; r < n + N; ++r)
      if (!ms_finite(d.ms[r])) err |= ISD_DEV_NONFINITE;
    int a = 0;
    for (int j = 0; j < kMaxN; ++j) d.px[j] = NAN;
    if (!err) {
      for (int j = 1; j <= n; ++j) {
        const float px = prob_of(s_lx[j - 1], d.ms[j - 1].x, d.ms[j - 1].y);
        d.px[j - 1] = px;
        // u * q < p compared exactly (fp32 operands, exact fp64 product).
        if (static_cast<double>(d.u[j]) * static_cast<double>(s_qx[j - 1]) < static_cast<double>(px))
          ++a;
        else
          break;
      }
    }
    d.n = n;
    d.a = a;
    d.err = err;
  }
  __syncthreads();
}

// ================================================================ outputs
// The outputs of sequence b that the decision alone fixes (all of them on
// an error). What depends on a draw is written by the workgroup that makes
// it: emit[a] (the bonus or the residual draw), the new drafts and their
// q(x), the residual mass.
__device__ __forceinline__ void write_decided(const AcceptParams& p, int b, const Decision& d) {
  const int N = p.N, nd = N - 1, n = d.n, a = d.a;
  if (d.err) {
    p.accepted[b] = -1;
    p.n_emit[b] = 0;
    p.kv_commit[b] = 0;
    for (int k = 0; k < N; ++k) p.emit[b * N + k] = -1;
    p.out.n_draft[b] = p.in.n_draft[b];
    p.out.q_row[b] = p.in.q_row[b];
    for (int k = 0; k < nd; ++k) {
      p.out.drafts[b * nd + k] = p.in.drafts[b * nd + k];
      p.out.q_x[b * nd + k] = p.in.q_x[b * nd + k];
      p.out.q_m[b * nd + k] = p.in.q_m[b * nd + k];
      p.out.q_s[b * nd + k] = p.in.q_s[b * nd + k];
    }
    if (p.resid_mass) p.resid_mass[b] = -1.f;
    if (p.p_x)
      for (int k = 0; k < nd; ++k) p.p_x[b * nd + k] = NAN;
    if (p.row_m)
      for (int r = 0; r < p.rows; ++r) {
        p.row_m[b * p.rows + r] = NAN;
        p.row_s[b * p.rows + r] = NAN;
      }
    set_dev_err(p.dev_err, static_cast<uint32_t>(d.err));
    return;
  }
  p.accepted[b] = a;
  p.n_emit[b] = a + 1;
  p.kv_commit[b] = a + 1;
  if (p.ctx) p.ctx[b] += a + 1;
  for (int k = 0; k < N; ++k)
    if (k != a) p.emit[b * N + k] = k < a ? p.in.drafts[b * nd + k] : -1;
  if (a == n) {
    p.out.n_draft[b] = nd;
    p.out.q_row[b] = n + 1;
    for (int k = 1; k <= nd; ++k) {
      p.out.q_m[b * nd + k - 1] = d.ms[n + k].x;
      p.out.q_s[b * nd + k - 1] = d.ms[n + k].y;
    }
    if (p.resid_mass) p.resid_mass[b] = -1.f;
  } else {
    p.out.n_draft[b] = 0;
    p.out.q_row[b] = 0;
    for (int k = 0; k < nd; ++k) {
      p.out.drafts[b * nd + k] = -1;
      p.out.q_x[b * nd + k] = 0.f;
      p.out.q_m[b * nd + k] = 0.f;
      p.out.q_s[b * nd + k] = 0.f;
    }
  }
  if (p.p_x)
    for (int k = 0; k < nd; ++k) p.p_x[b * nd + k] = d.px[k];
  if (p.row_m)
    for (int r = 0; r < p.rows; ++r) {
      const bool rd = r < n + N;
      p.row_m[b * p.rows + r] = rd ? d.ms[r].x : NAN;
      p.row_s[b * p.rows + r] = rd ? d.ms[r].y : NAN;
    }
}

// =========================================================== decide kernel
template <typename E>
__global__ __launch_bounds__(kThreads) void accept_decide_kernel(AcceptParams p) {
  const int slice = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ Decision d;
  decide<E>(p, b, d);
  const int n = d.n, a = d.a, N = p.N, nd = N - 1;
  if (slice == 0 && tid == 0) write_decided(p, b, d);
  if (d.err) return;
  const int nres = (p.nch + kResidChunks - 1) / kResidChunks;  // residual slices
  if (slice >= (a == n ? N : nres)) return;
  if (a == n) {
    // Every draft passed. Slice 0 draws the bonus from row n, slice k
    // proposal k from row n + k; each writes its own outputs.
    const int r = n + slice;
    int tok;
    float q;
    if (p.argmax && slice > 0) {
      tok = argmax_row<E>(p, b, r, d.st[r], d.ms[r].x);
      q = 1.f;
    } else {
      tok = sample_row<E>(p, b, r, d.st[r], d.ms[r].x, d.ms[r].y, d.u[N + slice], &q);
    }
    if (tid == 0) {
      if (slice == 0) {
        p.emit[b * N + a] = tok;
      } else {
        p.out.drafts[b * nd + slice - 1] = tok;
        p.out.q_x[b * nd + slice - 1] = q;
      }
    }
    return;
  }
  // Draft a+1 was rejected: residual sums of chunks kResidChunks * slice ..
  __shared__ ResidArgs s_ra;
  if (tid == 0) {
    ResidArgs ra;
    ra.a = a;
    ra.Ma = d.ms[a].x;
    ra.Sa = d.ms[a].y;
    ra.qm = p.in.q_m[b * nd + a];
    ra.qs = p.in.q_s[b * nd + a];
    ra.qrow = d.qrow;
    ra.x_rej = p.in.drafts[b * nd + a];
    s_ra = ra;
  }
  __syncthreads();
  {
    const ResidArgs ra = s_ra;
    ResidWeights<E> wf[kResidChunks];
#pragma unroll
    for (int h = 0; h < kResidChunks; ++h) {
      const int c = kResidChunks * slice + h;
      if (c < p.nch) wf[h] = resid_weights<E>(p, b, ra, c);  // both chunks' loads in flight together
    }
#pragma unroll
    for (int h = 0; h < kResidChunks; ++h) {
      const int c = kResidChunks * slice + h;
      if (c < p.nch) {
        float local = 0.f;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) local += wf[h](k);
        const float tot = block_sum(local);
        if (tid == 0) put_f32(&p.resid[static_cast<long>(b) * p.nch + c], tot);
      }
    }
  }
  // Arrival: thread 0 made this workgroup's stores; once they are complete
  // it counts the workgroup in. The one that brings the count to nres
  // reads every slice's sums with device-coherent loads, picks the chunk
  // and rescans it.
  __shared__ int s_last;
  if (tid == 0) {
    stores_done();
    s_last = __hip_atomic_fetch_add(&p.arrive[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nres - 1;
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  if (!s_last) return;
  __shared__ float s_res[kMaxChunks];
  __shared__ float s_mass, s_trel;
  __shared__ int s_c;
  if (tid < p.nch) s_res[tid] = get_f32(&p.resid[static_cast<long>(b) * p.nch + tid]);
  __syncthreads();
  if (tid == 0) {
    float W = 0.f;
    for (int c = 0; c < p.nch; ++c) W += s_res[c];
    s_mass = W;
    const float t = d.u[N] * W;
    float run = 0.f, trel = INFINITY;
    int c_sel = -1, last_nz = 0;
    for (int c = 0; c < p.nch; ++c) {
      const float wc = s_res[c];
      if (wc > 0.f) last_nz = c;
      if (c_sel < 0 && run + wc > t) {
        c_sel = c;
        trel = t - run;
      }
      run += wc;
    }
    s_c = c_sel >= 0 ? c_sel : last_nz;
    s_trel = c_sel >= 0 ? trel : INFINITY;
  }
  __syncthreads();
  int tok;
  if (s_mass > 0.f) {
    ResidWeights<E> wf = resid_weights<E>(p, b, s_ra, s_c);
    float w;
    tok = chunk_search(wf, s_c, s_trel, &w);
  } else {
    // No residual mass left (P_a <= Q_{a+1} everywhere): draw from P_a.
    float q;
    tok = sample_row<E>(p, b, a, d.st[a], d.ms[a].x, d.ms[a].y, d.u[N], &q);
  }
  if (tid == 0) {
    p.emit[b * N + a] = tok;
    if (p.resid_mass) p.resid_mass[b] = s_mass;
  }
}

// ----------------------------------------------------------- block assembly
// The next step's stride block: row 0 is the newest emitted token (the bonus
// or the resampled one, at position ctx after the commit), rows 1..n the n
// pending drafts, the rest MASK. One thread per (sequence, row).
__global__ __launch_bounds__(256) void block_assemble_kernel(const int32_t* n_draft, const int32_t* drafts,
                                                             const int32_t* emit, const int32_t* n_emit,
                                                             const int32_t* ctx, int C, int N, int32_t mask_id,
                                                             int32_t* tokens, int32_t* positions, uint8_t* is_mask,
                                                             int32_t* dev_err) {
  const int R = 2 * N;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= C * R) return;
  const int b = idx / R, i = idx % R;
  const int n = n_draft[b], ne = n_emit[b];
  const bool ok = (n == 0 || n == N - 1) && ne >= 1 && ne <= N;
  int32_t tok = -1;
  bool masked = false;
  if (!ok) {
    if (i == 0) set_dev_err(dev_err, ISD_DEV_STATE);
  } else if (i == 0) {
    tok = emit[static_cast<long>(b) * N + ne - 1];
  } else if (i <= n) {
    tok = drafts[static_cast<long>(b) * (N - 1) + i - 1];
  } else {
    tok = mask_id;
    masked = true;
  }
  tokens[idx] = tok;
  if (is_mask) is_mask[idx] = masked ? 1 : 0;
  if (positions) positions[idx] = ctx[b] + i;
}

}  // namespace isd

// The workspace of isd_accept_noalloc: a fixed array in device memory, one
// copy per GPU, kept until the process ends. In host code its name is only a
// stand-in: the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// ================================================================ host API
namespace {
using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

size_t up256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct AcceptLayout {
  int nch, ns;
  size_t stats_off, lx_off, resid_off, arrive_off, total;
};

AcceptLayout accept_layout(int C, int N, int V, int rows) {
  AcceptLayout L;
  L.nch = (V + kChunk - 1) / kChunk;
  const int nres = (L.nch + kResidChunks - 1) / kResidChunks;
  L.ns = nres > N ? nres : N;
  L.stats_off = 0;
  L.lx_off = up256(static_cast<size_t>(C) * rows * L.nch * sizeof(float2));
  L.resid_off = L.lx_off + up256(static_cast<size_t>(C) * kMaxN * sizeof(float));
  L.arrive_off = L.resid_off + up256(static_cast<size_t>(C) * L.nch * sizeof(float));
  L.total = L.arrive_off + up256(static_cast<size_t>(C) * sizeof(int));
  return L;
}

bool state_ok(const isd_seq_state& s) { return s.n_draft && s.drafts && s.q_x && s.q_m && s.q_s && s.q_row; }

template <typename E>
hipError_t launch_accept(const AcceptParams& p, bool stats_given, hipStream_t stream) {
  if (stats_given) {
    const int threads = p.C * (p.N - 1);
    hipLaunchKernelGGL(accept_prep_kernel<E>, dim3((threads + 255) / 256), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(accept_stats_kernel<E>, dim3(p.nch, 2 * p.N - 1, p.C), dim3(kThreads), 0, stream, p);
  }
  hipLaunchKernelGGL(accept_decide_kernel<E>, dim3(p.ns, p.C), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

extern "C" {

size_t isd_accept_workspace_size(int C, int N, int V, int rows) {
  if (C < 0 || N < 2 || N > kMaxN || V < 1 || V > kMaxChunks * kChunk || rows < 2 * N - 1) return 0;
  return accept_layout(C, N, V, rows).total;
}

}  // extern "C"

namespace {

// isd_accept with the workspace given separately (ws_bytes 0: none).
int accept_with_workspace(const isd_accept_args* a, void* ws_ptr, size_t ws_bytes, hipStream_t stream) {
  if (!a) return ISD_E_INVALID;
  if (a->C < 0 || a->N < 2 || a->V < 1) return ISD_E_INVALID;
  if (a->C > 65535) return ISD_E_UNSUPPORTED;  // sequences map to a grid dimension
  if (a->N > kMaxN) return ISD_E_UNSUPPORTED;
  if (a->V > kMaxChunks * kChunk) return ISD_E_UNSUPPORTED;  // chunk statistics are cached in LDS
  if (a->rows < 2 * a->N - 1) return ISD_E_INVALID;
  if (a->dtype != ISD_BF16 && a->dtype != ISD_F32) return ISD_E_UNSUPPORTED;
  if (a->proposal != ISD_PROPOSE_SAMPLE && a->proposal != ISD_PROPOSE_ARGMAX) return ISD_E_INVALID;
  if (a->C == 0) return ISD_OK;
  if (!a->logits || !state_ok(a->in) || !state_ok(a->out)) return ISD_E_INVALID;
  if (!a->accepted || !a->n_emit || !a->emit || !a->kv_commit) return ISD_E_INVALID;
  if ((a->row_m == nullptr) != (a->row_s == nullptr)) return ISD_E_INVALID;
  const int esz = a->dtype == ISD_BF16 ? 2 : 4;
  if (a->ld < a->V || (a->ld * esz) % 16 != 0) return ISD_E_INVALID;
  if (!aligned16(a->logits) || (a->prev_logits && !aligned16(a->prev_logits))) return ISD_E_INVALID;
  if (reinterpret_cast<uintptr_t>(a->chunk_stats) & 7u) return ISD_E_INVALID;  // read as float pairs
  if (a->in.n_draft == a->out.n_draft || a->in.drafts == a->out.drafts || a->in.q_x == a->out.q_x ||
      a->in.q_m == a->out.q_m || a->in.q_s == a->out.q_s || a->in.q_row == a->out.q_row)
    return ISD_E_INVALID;
  const AcceptLayout L = accept_layout(a->C, a->N, a->V, a->rows);
  if (!ws_ptr || ws_bytes < L.total || !aligned16(ws_ptr)) return ISD_E_WORKSPACE;
  int rc = isd_check_device_internal();
  if (rc) return rc;

  AcceptParams p;
  p.logits = a->logits;
  p.prev_logits = a->prev_logits;
  p.ld = static_cast<long>(a->ld);
  p.C = a->C;
  p.N = a->N;
  p.V = a->V;
  p.rows = a->rows;
  p.nch = L.nch;
  p.ns = L.ns;
  p.in = a->in;
  p.out = a->out;
  p.seed = a->seed;
  p.step = a->step;
  p.step_dev = a->step_dev;
  p.accepted = a->accepted;
  p.n_emit = a->n_emit;
  p.emit = a->emit;
  p.kv_commit = a->kv_commit;
  p.ctx = a->ctx;
  p.p_x = a->p_x;
  p.resid_mass = a->resid_mass;
  p.row_m = a->row_m;
  p.row_s = a->row_s;
  char* ws = static_cast<char*>(ws_ptr);
  const bool given = a->chunk_stats != nullptr;
  p.stats = given ? reinterpret_cast<float2*>(const_cast<float*>(a->chunk_stats))
                  : reinterpret_cast<float2*>(ws + L.stats_off);
  p.lx = reinterpret_cast<float*>(ws + L.lx_off);
  p.resid = reinterpret_cast<float*>(ws + L.resid_off);
  p.arrive = reinterpret_cast<int*>(ws + L.arrive_off);
  p.argmax = a->proposal == ISD_PROPOSE_ARGMAX;
  p.dev_err = a->dev_err;
  const hipError_t e =
      a->dtype == ISD_BF16 ? launch_accept<uint16_t>(p, given, stream) : launch_accept<float>(p, given, stream);
  return e == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

// ------------------------------------------------- allocation-free variant
std::mutex g_scratch_mutex;
void* g_scratch_ptr[64];

// Device address of `scratch` on the current device, or null.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int isd_accept(const isd_accept_args* a, hipStream_t stream) {
  if (!a) return ISD_E_INVALID;
  return accept_with_workspace(a, a->ws, a->ws_bytes, stream);
}

size_t isd_accept_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

int isd_accept_noalloc(const isd_accept_args* a, hipStream_t stream) {
  if (!a) return ISD_E_INVALID;
  const size_t need = isd_accept_workspace_size(a->C, a->N, a->V, a->rows);
  if (need > kNoAllocScratchBytes) return ISD_E_WORKSPACE;  // beyond the fixed scratch
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  void* ws = scratch_address();
  if (!ws) return ISD_E_LAUNCH;
  return accept_with_workspace(a, ws, kNoAllocScratchBytes, stream);
}

int isd_block_assemble(const isd_seq_state* st, const int32_t* emit, const int32_t* n_emit, const int32_t* ctx,
                       int C, int N, int32_t mask_id, int32_t* tokens, int32_t* positions, uint8_t* is_mask,
                       int32_t* dev_err, hipStream_t stream) {
  if (!st || C < 0 || N < 2) return ISD_E_INVALID;
  if (N > kMaxN) return ISD_E_UNSUPPORTED;
  if (C == 0) return ISD_OK;
  if (!st->n_draft || !st->drafts || !emit || !n_emit || !tokens) return ISD_E_INVALID;
  if (positions && !ctx) return ISD_E_INVALID;
  if (static_cast<long>(C) * 2 * N > INT_MAX) return ISD_E_UNSUPPORTED;
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  const int total = C * 2 * N;
  hipLaunchKernelGGL(block_assemble_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, st->n_draft, st->drafts,
                     emit, n_emit, ctx, C, N, mask_id, tokens, positions, is_mask, dev_err);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // extern "C"

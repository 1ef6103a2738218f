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
// Two launches, both HBM-streaming and deterministic:
//   stats   one pass over every logits row the step may read: per 8192-entry
//           chunk, the max and sum of exp(l - max) (fp32 from exact bf16);
//           a workgroup takes two chunks with all their loads in flight.
//   sample  grid (slices, sequences). Every workgroup rebuilds the row
//           statistics and the accept decision from the chunk stats (same
//           fixed-order arithmetic, so all agree). On a rejection each slice
//           sums the residual max(0, P_a - Q_{a+1}) over its chunk; when all
//           drafts pass, slice k rescans the one chunk where the CDF of row
//           n + k crosses its uniform (bonus for k = 0, proposals after).
//           The last workgroup of a sequence to finish (a counter per
//           sequence, zeroed by the stats launch) then picks and rescans the
//           residual chunk and writes the outputs and the next state.
// When the caller passes the chunk statistics (isd_lm_head wrote them with
// the logits), a small launch that zeroes the counters replaces the stats
// launch.
#include "isd_common.hpp"

namespace isd {

constexpr int kChunk = kVocabChunk;  // vocab entries per stats chunk
constexpr int kThreads = 256;    // threads per workgroup
constexpr int kPerThread = 32;   // entries per thread in a chunk
constexpr int kStatsChunks = 2;  // chunks per workgroup of the stats launch
constexpr int kMaxN = 8;
constexpr int kMaxChunks = 64;   // vocabularies up to 524,288 entries
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
  float2* stats;    // [C][rows][nch] (chunk max, chunk sum)
  float* resid;     // [C][nch] residual sum per chunk
  int2* samp;       // [C][N] (token, bits of q(x)) from the sample kernel
  int* arrive;      // [C] workgroups of the sample launch done, per sequence
  int32_t* dev_err;
  int argmax;       // proposals are argmax q (a point mass at the draft)
  int stats_given;  // stats come from the caller (isd_lm_head): no statistics pass
};

// ------------------------------------------- values handed between workgroups
// The slice results of the sample launch reach the sequence's last
// workgroup through device-coherent (agent-scope) atomic stores and loads,
// so no cache-wide writeback or invalidate is needed: the writer waits for
// its store to complete before it counts itself in.
__device__ __forceinline__ void put_f32(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_f32(float* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_sample(int2* ptr, int tok, float q) {
  const unsigned long long v =
      static_cast<unsigned long long>(static_cast<uint32_t>(tok)) | (static_cast<unsigned long long>(__float_as_uint(q)) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(ptr), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int2 get_sample(int2* ptr) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<unsigned long long*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_int2(static_cast<int>(static_cast<uint32_t>(v)), static_cast<int>(static_cast<uint32_t>(v >> 32)));
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

// Load this thread's 32 entries of chunk c (entries >= V become -inf).
template <typename E>
__device__ __forceinline__ void load_chunk_slice(const E* row, int V, int c, float (&x)[kPerThread]) {
  constexpr int KP = Elem<E>::kPerVec;
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
#pragma unroll
  for (int q = 0; q < kPerThread / KP; ++q) {
    const int vq = v0 + q * KP;
    if (vq + KP <= V) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + vq);
      float f[KP];
      unpack16(w, f);
#pragma unroll
      for (int k = 0; k < KP; ++k) x[q * KP + k] = f[k];
    } else {
#pragma unroll
      for (int k = 0; k < KP; ++k) x[q * KP + k] = (vq + k < V) ? load_elem(row, vq + k) : -INFINITY;
    }
  }
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

// ============================================================ stats kernel
// Entries c*kChunk + i*2048 + 8t .. +7 (i = 0..3) of chunk c go to thread t:
// each load instruction of the workgroup reads 4 KB of contiguous logits.
// (A chunk's max and sum do not depend on which thread holds what; the
// sampling rescans keep token order per thread.)
template <typename E>
__device__ __forceinline__ void load_chunk_coalesced(const E* row, int V, int c, float (&x)[kPerThread]) {
  constexpr int KP = Elem<E>::kPerVec;  // 8 bf16 or 4 fp32 per 16 bytes
#pragma unroll
  for (int q = 0; q < kPerThread / KP; ++q) {
    const int vq = c * kChunk + q * kThreads * KP + threadIdx.x * KP;
    if (vq + KP <= V) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + vq);
      float f[KP];
      unpack16(w, f);
#pragma unroll
      for (int k = 0; k < KP; ++k) x[q * KP + k] = f[k];
    } else {
#pragma unroll
      for (int k = 0; k < KP; ++k) x[q * KP + k] = (vq + k < V) ? load_elem(row, vq + k) : -INFINITY;
    }
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(AcceptParams p) {
  const int c0 = blockIdx.x * kStatsChunks, r = blockIdx.y, b = blockIdx.z;
  if (c0 == 0 && r == 0 && threadIdx.x == 0) p.arrive[b] = 0;  // the sample launch counts from zero
  int n = p.in.n_draft[b];
  n = n < 0 ? 0 : (n > p.N - 1 ? p.N - 1 : n);
  if (r > n + p.N - 1) return;
  const E* row = row_ptr<E>(p.logits, p.ld, p.rows, b, r);
  float x[kStatsChunks][kPerThread];
#pragma unroll
  for (int h = 0; h < kStatsChunks; ++h) {
    if (c0 + h < p.nch) {
      load_chunk_coalesced<E>(row, p.V, c0 + h, x[h]);
    } else {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) x[h][k] = -INFINITY;
    }
  }
#pragma unroll
  for (int h = 0; h < kStatsChunks; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) m = fmaxf(m, x[h][k]);
    float s = 0.f;
    if (m != -INFINITY) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) s += weight_of(x[h][k], ml);
    }
    block_reduce_ms(m, s);
    if (threadIdx.x == 0 && c0 + h < p.nch) p.stats[(static_cast<long>(b) * p.rows + r) * p.nch + c0 + h] = make_float2(m, s);
  }
}

// With the chunk statistics given, only the arrival counters of the sample
// launch need clearing.
__global__ __launch_bounds__(256) void accept_arrive_reset_kernel(int* arrive, int C) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < C) arrive[b] = 0;
}

// ------------------------------------------------ shared per-sequence logic
struct Decision {
  int n, a, err;                     // err: ISD_DEV_* bits, 0 if the step can be taken
  int qrow;                          // first row of the previous step that proposed
  float M[2 * kMaxN];                // row max
  float S[2 * kMaxN];                // row sum exp(l - M)
  float u[2 * kMaxN];                // uniforms by slot
  float px[kMaxN];                   // P_{j-1}(x_j) of tested drafts
  int draft[kMaxN];                  // pending draft ids
  float2 st[2 * kMaxN][kMaxChunks];  // chunk (max, sum) of the rows read
};

// Rebuild row statistics, uniforms and the accept decision of sequence b.
// Every workgroup that calls this computes the same values. The state, the
// chunk statistics of every row and the uniforms are fetched together; the
// logits of the drafts follow in one more round trip. Result in LDS.
template <typename E>
__device__ void decide(const AcceptParams& p, int b, Decision& d) {
  const int tid = threadIdx.x;
  const int N = p.N, nd = N - 1, R = 2 * N - 1;
  __shared__ int s_n, s_draft[kMaxN];
  __shared__ float s_qx[kMaxN], s_pall[kMaxN];
  if (tid == 0) {
    s_n = p.in.n_draft[b];
    d.qrow = p.in.q_row[b];
  }
  if (tid < nd) {
    s_draft[tid] = p.in.drafts[b * nd + tid];
    s_qx[tid] = p.in.q_x[b * nd + tid];
    d.draft[tid] = s_draft[tid];
  }
  for (int i = tid; i < R * p.nch; i += kThreads)
    d.st[i / p.nch][i % p.nch] = p.stats[(static_cast<long>(b) * p.rows + i / p.nch) * p.nch + i % p.nch];
  if (tid < 2 * N) {
    const uint64_t step = p.step_dev ? *p.step_dev : p.step;
    d.u[tid] = uniform_of(philox_word0(static_cast<uint64_t>(tid), static_cast<uint64_t>(b), step, 0ull, p.seed, 0ull));
  }
  __syncthreads();
  // every thread clamps n the same way; thread 0 records what was wrong
  const int n_raw = s_n;
  const int n = (n_raw < 0 || n_raw > nd) ? 0 : n_raw;
  if (tid == 0) {
    int err = 0;
    if (n_raw < 0 || n_raw > nd) err |= ISD_DEV_STATE;
    if (n > 0 && ((!p.argmax && !p.prev_logits) || d.qrow < 0 || d.qrow + n - 1 >= p.rows)) err |= ISD_DEV_STATE;
    for (int j = 0; j < n; ++j)
      if (s_draft[j] < 0 || s_draft[j] >= p.V) err |= ISD_DEV_TOKEN_OOB;
    d.n = n;
    d.err = err;
  }
  // the logit of draft j+1 in verify row j (loaded before the row sums exist)
  float lx = 0.f;
  const bool draft_ok = tid < n && s_draft[tid] >= 0 && s_draft[tid] < p.V;
  if (draft_ok) lx = load_elem(row_ptr<E>(p.logits, p.ld, p.rows, b, tid), s_draft[tid]);
  const int nrows = n + N;  // rows 0 .. n + N - 1
  __syncthreads();
  if (tid < nrows) {
    float M = -INFINITY;
    for (int c = 0; c < p.nch; ++c) M = fmaxf(M, d.st[tid][c].x);
    float S = 0.f;
    if (M != -INFINITY) {
      for (int c = 0; c < p.nch; ++c) S += d.st[tid][c].y * fast_exp2((d.st[tid][c].x - M) * kLog2e);
    }
    d.M[tid] = M;
    d.S[tid] = S;
    if (!(M > -INFINITY && M < INFINITY && S > 0.f && S < INFINITY)) atomicOr(&d.err, static_cast<int>(ISD_DEV_NONFINITE));
  }
  __syncthreads();
  if (tid < n) s_pall[tid] = draft_ok ? prob_of(lx, d.M[tid], d.S[tid]) : NAN;
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    for (int j = 0; j < kMaxN; ++j) d.px[j] = NAN;
    if (!d.err) {
      for (int j = 1; j <= n; ++j) {
        const float px = s_pall[j - 1];
        d.px[j - 1] = px;
        // u * q < p compared exactly (fp32 operands, exact fp64 product).
        if (static_cast<double>(d.u[j]) * static_cast<double>(s_qx[j - 1]) < static_cast<double>(px))
          ++a;
        else
          break;
      }
    }
    d.a = a;
  }
  __syncthreads();
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

// Inverse-CDF search inside one chunk: weights w[] of this thread's 32
// entries (thread order = token order), target t_rel measured from the start
// of the chunk. Returns the smallest crossing token id, or the last token
// with non-zero weight in the chunk when rounding leaves no crossing.
__device__ int chunk_search(const float (&w)[kPerThread], int c, float t_rel) {
  __shared__ int s_tok, s_last;
  if (threadIdx.x == 0) {
    s_tok = 0x7fffffff;
    s_last = -1;
  }
  float local = 0.f;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) local += w[k];
  const float base = block_exclusive_scan(local);  // also syncs
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
  const float tr = t_rel - base;
  if (tr >= 0.f && local > tr) {
    float acc = 0.f;
    int hit = -1;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      acc += w[k];
      if (hit < 0 && acc > tr) hit = v0 + k;
    }
    if (hit >= 0) atomicMin(&s_tok, hit);
  }
  int last = -1;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (w[k] > 0.f) last = v0 + k;
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  const int tok = s_tok != 0x7fffffff ? s_tok : s_last;
  __syncthreads();
  return tok;
}

// Choose the chunk of a row whose (rescaled) chunk sums cross u * S.
// Returns the chunk and writes the target relative to its start.
__device__ __forceinline__ int pick_chunk_from_stats(const float2 (&st)[kMaxChunks], int nch, float M, float t,
                                                     float* t_rel) {
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

// Sample from softmax(row r) with uniform u: returns the token.
template <typename E>
__device__ int sample_row(const AcceptParams& p, const Decision& d, int b, int r, float u) {
  const float M = d.M[r], S = d.S[r];
  float t_rel;
  const int c = pick_chunk_from_stats(d.st[r], p.nch, M, u * S, &t_rel);
  float x[kPerThread];
  load_chunk_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, r), p.V, c, x);
  const float ml = M * kLog2e;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) x[k] = weight_of(x[k], ml);
  return chunk_search(x, c, t_rel);
}

// argmax of row r, ties to the smallest id: the first chunk whose maximum is
// the row maximum holds it; its entries are compared exactly with that value.
template <typename E>
__device__ int argmax_row(const AcceptParams& p, const Decision& d, int b, int r) {
  __shared__ int s_tok;
  const float M = d.M[r];
  int c = 0;
  while (c + 1 < p.nch && d.st[r][c].x != M) ++c;
  if (threadIdx.x == 0) s_tok = 0x7fffffff;
  __syncthreads();
  float x[kPerThread];
  load_chunk_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, r), p.V, c, x);
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
  int hit = 0x7fffffff;
#pragma unroll
  for (int k = kPerThread - 1; k >= 0; --k)
    if (x[k] == M) hit = v0 + k;
  if (hit != 0x7fffffff) atomicMin(&s_tok, hit);
  __syncthreads();
  const int tok = s_tok;
  __syncthreads();
  return tok;
}

// Residual weights of this thread's slice of chunk c. With argmax proposals
// Q_{a+1} is a point mass at the rejected draft: the residual is P_a with
// that token removed, and the previous block is not read.
template <typename E>
__device__ __forceinline__ void resid_slice(const AcceptParams& p, int b, const Decision& d, int c,
                                            float (&w)[kPerThread]) {
  const int a = d.a;
  float x[kPerThread], y[kPerThread];
  load_chunk_slice<E>(row_ptr<E>(p.logits, p.ld, p.rows, b, a), p.V, c, x);
  if (p.argmax) {
    const float ma_l2 = d.M[a] * kLog2e, inv_sa = 1.f / d.S[a];
    const int x_rej = d.draft[a], v0 = c * kChunk + threadIdx.x * kPerThread;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
#pragma clang fp contract(off)
      const float pa = weight_of(x[k], ma_l2) * inv_sa;
      w[k] = (x[k] == -INFINITY || v0 + k == x_rej) ? 0.f : pa;
    }
    return;
  }
  const int qrow = d.qrow + a;
  load_chunk_slice<E>(row_ptr<E>(p.prev_logits, p.ld, p.rows, b, qrow), p.V, c, y);
  const float ma_l2 = d.M[a] * kLog2e, inv_sa = 1.f / d.S[a];
  const float mq_l2 = p.in.q_m[b * (p.N - 1) + a] * kLog2e, inv_sq = 1.f / p.in.q_s[b * (p.N - 1) + a];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) w[k] = (x[k] == -INFINITY) ? 0.f : resid_weight(x[k], y[k], ma_l2, inv_sa, mq_l2, inv_sq);
}

// ====================================================== finish (one WG)
// Outputs and next state of sequence b, run by the last workgroup of the
// sample launch to finish for it: the residual chunk is picked from the
// slice sums and rescanned here.
template <typename E>
__device__ void finish(const AcceptParams& p, int b, const Decision& d) {
  const int N = p.N, nd = N - 1;
  const int tid = threadIdx.x;
  if (d.err) {
    if (tid == 0) {
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
    }
    return;
  }
  const int n = d.n, a = d.a;
  __shared__ int s_t;
  __shared__ float s_mass;
  // the other workgroups' results, fetched in parallel
  __shared__ float s_res[kMaxChunks];
  __shared__ int2 s_smp[kMaxN];
  if (a < n) {
    if (tid < p.nch) s_res[tid] = get_f32(&p.resid[static_cast<long>(b) * p.nch + tid]);
  } else if (tid < N) {
    s_smp[tid] = get_sample(&p.samp[b * N + tid]);
  }
  __syncthreads();
  if (a < n) {
    // Residual: pick the chunk from the per-chunk sums, rescan it.
    if (tid == 0) {
      float W = 0.f;
      for (int c = 0; c < p.nch; ++c) W += s_res[c];
      s_mass = W;
    }
    __syncthreads();
    const float W = s_mass;
    int tok;
    if (W > 0.f) {
      const float t = d.u[N] * W;
      __shared__ int s_c;
      __shared__ float s_trel;
      if (tid == 0) {
        float run = 0.f;
        int c_sel = -1, last_nz = 0;
        float trel = INFINITY;
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
      float w[kPerThread];
      resid_slice<E>(p, b, d, s_c, w);
      tok = chunk_search(w, s_c, s_trel);
    } else {
      // No residual mass left (P_a <= Q_{a+1} everywhere): draw from P_a.
      tok = sample_row<E>(p, d, b, a, d.u[N]);
    }
    if (tid == 0) s_t = tok;
  } else {
    if (tid == 0) s_t = s_smp[0].x;
  }
  __syncthreads();
  if (tid == 0) {
    const int t = s_t;
    p.accepted[b] = a;
    p.n_emit[b] = a + 1;
    p.kv_commit[b] = a + 1;
    if (p.ctx) p.ctx[b] += a + 1;
    for (int k = 0; k < N; ++k) {
      int v = -1;
      if (k < a) v = p.in.drafts[b * nd + k];
      if (k == a) v = t;
      p.emit[b * N + k] = v;
    }
    if (a == n) {
      p.out.n_draft[b] = nd;
      p.out.q_row[b] = n + 1;
      for (int k = 1; k <= nd; ++k) {
        const int2 sp = s_smp[k];
        p.out.drafts[b * nd + k - 1] = sp.x;
        p.out.q_x[b * nd + k - 1] = __int_as_float(sp.y);
        p.out.q_m[b * nd + k - 1] = d.M[n + k];
        p.out.q_s[b * nd + k - 1] = d.S[n + k];
      }
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
    if (p.resid_mass) p.resid_mass[b] = (a < n) ? s_mass : -1.f;
    if (p.p_x)
      for (int k = 0; k < nd; ++k) p.p_x[b * nd + k] = d.px[k];
    if (p.row_m)
      for (int r = 0; r < p.rows; ++r) {
        const bool rd = r < n + N;
        p.row_m[b * p.rows + r] = rd ? d.M[r] : NAN;
        p.row_s[b * p.rows + r] = rd ? d.S[r] : NAN;
      }
  }
}

// =========================================================== sample kernel
template <typename E>
__global__ __launch_bounds__(kThreads) void accept_sample_kernel(AcceptParams p) {
  const int slice = blockIdx.x, b = blockIdx.y;
  __shared__ Decision d;
  decide<E>(p, b, d);
  const int n = d.n, a = d.a;
  if (!d.err) {
    if (a < n) {
      // residual sums of chunks kStatsChunks * slice ..
#pragma unroll
      for (int h = 0; h < kStatsChunks; ++h) {
        const int c = kStatsChunks * slice + h;
        if (c < p.nch) {
          float w[kPerThread];
          resid_slice<E>(p, b, d, c, w);
          float local = 0.f;
#pragma unroll
          for (int k = 0; k < kPerThread; ++k) local += w[k];
          const float tot = block_sum(local);
          if (threadIdx.x == 0) put_f32(&p.resid[static_cast<long>(b) * p.nch + c], tot);
        }
      }
    } else if (slice < p.N) {
      const int r = n + slice;  // slice 0: bonus row n; slice k: proposal row n + k
      if (p.argmax && slice > 0) {
        const int tok = argmax_row<E>(p, d, b, r);
        if (threadIdx.x == 0) put_sample(&p.samp[b * p.N + slice], tok, 1.f);
      } else {
        const int tok = sample_row<E>(p, d, b, r, d.u[p.N + slice]);
        if (threadIdx.x == 0) {
          const float l = load_elem(row_ptr<E>(p.logits, p.ld, p.rows, b, r), tok);
          put_sample(&p.samp[b * p.N + slice], tok, prob_of(l, d.M[r], d.S[r]));
        }
      }
    }
  }
  // Arrival: thread 0 made this workgroup's stores; once they are complete
  // (vmcnt 0) it counts the workgroup in. The one that brings the count to
  // ns reads everybody's results with device-coherent loads.
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    // the compiler may not move the slice stores past the wait, nor the
    // counter update above it; the wait makes the stores complete first
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    s_last = __hip_atomic_fetch_add(&p.arrive[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.ns - 1;
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  if (!s_last) return;
  finish<E>(p, b, d);
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

// ================================================================ host API
namespace {
using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

struct AcceptLayout {
  int nch, ns;
  size_t stats_off, resid_off, samp_off, arrive_off, total;
};

AcceptLayout accept_layout(int C, int N, int V, int rows) {
  AcceptLayout L;
  L.nch = (V + kChunk - 1) / kChunk;
  const int pairs = (L.nch + kStatsChunks - 1) / kStatsChunks;
  L.ns = pairs > N ? pairs : N;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  L.stats_off = 0;
  L.resid_off = up(static_cast<size_t>(C) * rows * L.nch * sizeof(float2));
  L.samp_off = L.resid_off + up(static_cast<size_t>(C) * L.nch * sizeof(float));
  L.arrive_off = L.samp_off + up(static_cast<size_t>(C) * N * sizeof(int2));
  L.total = L.arrive_off + up(static_cast<size_t>(C) * sizeof(int));
  return L;
}

bool state_ok(const isd_seq_state& s) { return s.n_draft && s.drafts && s.q_x && s.q_m && s.q_s && s.q_row; }

template <typename E>
hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.stats_given)
    hipLaunchKernelGGL(accept_arrive_reset_kernel, dim3((p.C + 255) / 256), dim3(256), 0, stream, p.arrive, p.C);
  else
    hipLaunchKernelGGL(accept_stats_kernel<E>, dim3((p.nch + kStatsChunks - 1) / kStatsChunks, 2 * p.N - 1, p.C),
                       dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(accept_sample_kernel<E>, dim3(p.ns, p.C), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

extern "C" {

size_t isd_accept_workspace_size(int C, int N, int V, int rows) {
  if (C < 0 || N < 2 || N > kMaxN || V < 1 || V > kMaxChunks * kChunk || rows < 2 * N - 1) return 0;
  return accept_layout(C, N, V, rows).total;
}

int isd_accept(const isd_accept_args* a, hipStream_t stream) {
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
  if (!a->ws || a->ws_bytes < L.total || !aligned16(a->ws)) return ISD_E_WORKSPACE;
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
  char* ws = static_cast<char*>(a->ws);
  p.stats_given = a->chunk_stats != nullptr;
  p.stats = p.stats_given ? reinterpret_cast<float2*>(const_cast<float*>(a->chunk_stats))
                          : reinterpret_cast<float2*>(ws + L.stats_off);
  p.resid = reinterpret_cast<float*>(ws + L.resid_off);
  p.samp = reinterpret_cast<int2*>(ws + L.samp_off);
  p.arrive = reinterpret_cast<int*>(ws + L.arrive_off);
  p.argmax = a->proposal == ISD_PROPOSE_ARGMAX;
  p.dev_err = a->dev_err;
  const hipError_t e = a->dtype == ISD_BF16 ? launch_accept<uint16_t>(p, stream) : launch_accept<float>(p, stream);
  return e == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
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

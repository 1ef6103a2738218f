// Base projection GEMM and the gated LoRA of lossless R-ISD (gfx950).
//
// The adapter acts only at MASK positions so that clean positions keep the
// base model's outputs bit for bit (I-DLM, fr.news.hada.io, "Speedup Factor
// Explorer" and "Documentation et ressources > Lossless R-ISD"). Here that
// means: y = x W^T on every row with one fixed MFMA reduction order; MASK rows
// then get y + s * (x A^T) B^T, and clean rows keep the base value itself
// (selected, never recomputed).
//
// GEMM: y[M][Nout] fp32 = x[M][K] bf16 . W[Nout][K]^T bf16 ("NT": both
// operands K-contiguous). Four waves in a 2 x 2 grid, each TM x TN blocks of
// 32 x 32 (v_mfma_f32_32x32x16_bf16). K advances in slabs of 64 that travel
// from global memory straight into LDS (16-byte direct loads, XOR-swizzled
// rows, no register staging), three to five stages deep with one barrier per
// slab. The per-output reduction order is slab by slab in ascending K and
// does not depend on M, the tile choice, the other rows or the mask. A
// split-K launch runs the same loop over a fixed share of the slabs (the
// split count depends only on K).
// LM head: the same loop with an epilogue that stores bf16 logits and the
// per-row softmax statistics of each 128-column tile (isd_lm_head).
// LoRA: U = x A^T first, as a split-K GEMM whose partials are summed in
// split order. The delta U B^T of a 32x32 output block then runs on bf16
// MFMA with U split into bf16 high and low halves (about 16 mantissa bits):
// in the GEMM's epilogue for isd_linear_gated, in its own kernel for
// gated_lora_apply, with the same instruction sequence, so the two give the
// same bits.
#include <mutex>

#include "isd_common.hpp"

namespace isd {

constexpr int kBK = 64;
constexpr int kXcds = 8;  // XCDs of an MI355X

constexpr int kMaxSplits = 8;  // split-K shares of U = x A^T
constexpr int kMaxStages = 6;
constexpr int kLogitsTileN = 128;  // columns per tile of the LM head (TN = 2), a divisor of the vocabulary chunk
static_assert(kVocabChunk % kLogitsTileN == 0, "chunks are whole tiles");
constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU

// The LoRA delta of one 32x32 output block, U B^T, on bf16 MFMA: each U row
// (fp32) is split into a bf16 high part (truncation) and the bf16 rounding
// of the remainder, and the two halves run as two independent MFMA chains
// added at the end. Register e of lane (j, hh) is block row 8(e/4) + 4hh +
// e%4, column j. The GEMM epilogue and the stand-alone delta kernel both go
// through these two functions, so they produce the same bits.
template <int R16>
struct UFrag {
  bf16x8 hi[R16], lo[R16];
};

// Fragments of the U row this lane feeds to the MFMA (row = block row of
// lane32; hh selects the 8-entry half of each 16-entry step); null row:
// zeros.
template <int R16>
__device__ __forceinline__ UFrag<R16> u_frag(const float* row, int hh) {
  UFrag<R16> uf;
#pragma unroll
  for (int k = 0; k < R16; ++k) {
    f32x4 v0 = f32x4{}, v1 = f32x4{};
    if (row) {
      const f32x4* src = reinterpret_cast<const f32x4*>(row + 16 * k + 8 * hh);
      v0 = src[0];
      v1 = src[1];
    }
    const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    u32x4 hi, lo;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t ua = __float_as_uint(f[2 * t]) & 0xffff0000u, ub = __float_as_uint(f[2 * t + 1]) & 0xffff0000u;
      hi[t] = (ua >> 16) | ub;
      lo[t] = f32_to_bf16_bits(f[2 * t] - __uint_as_float(ua)) |
              (f32_to_bf16_bits(f[2 * t + 1] - __uint_as_float(ub)) << 16);
    }
    uf.hi[k] = __builtin_bit_cast(bf16x8, hi);
    uf.lo[k] = __builtin_bit_cast(bf16x8, lo);
  }
  return uf;
}

// The B^T operand of the delta for columns n0.. of B (bf16 [Nout][r]):
// lane (j, hh) holds B[n0 + j][16k + 8hh .. +8] for every 16-deep step k;
// columns past Nout give 0.
template <int R16>
struct BFrag {
  u32x4 v[R16];
};
template <int R16>
__device__ __forceinline__ BFrag<R16> b_frag(const uint16_t* B, int Nout, int n0, int lane32, int hh) {
  constexpr int r = 16 * R16;
  const int bcol = n0 + lane32;
  BFrag<R16> bf;
#pragma unroll
  for (int k = 0; k < R16; ++k)
    bf.v[k] = bcol < Nout ? *reinterpret_cast<const u32x4*>(B + static_cast<long>(bcol) * r + 16 * k + 8 * hh)
                          : u32x4{0, 0, 0, 0};
  return bf;
}

// U B^T of one 32x32 block from its fragments.
template <int R16>
__device__ __forceinline__ f32x16 lora_delta(const UFrag<R16>& uf, const BFrag<R16>& bf) {
  f32x16 dh = {}, dl = {};
#pragma unroll
  for (int k = 0; k < R16; ++k) {
    const bf16x8 bb = __builtin_bit_cast(bf16x8, bf.v[k]);
    dh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uf.hi[k], bb, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uf.lo[k], bb, dl, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) dh[e] += dl[e];
  return dh;
}

struct GemmParams {
  const uint16_t* x;    // [M][K]
  const uint16_t* w;    // [Nout][K]
  void* y;              // [splits][M][Nout]: fp32, or bf16 bits when ybf16
  int ybf16;            // store y rounded to bf16 (nearest even); never for split-K partials
  // gated epilogue (R16 > 0): MASK rows get y = acc + scale * U B^T
  const float* u;       // U = x A^T as u_splits split-K partials [u_splits][M][r] fp32
  int u_splits;         // summed in split order while staged into LDS
  const uint16_t* b;    // [Nout][r]
  const uint8_t* mask;  // [M]
  float scale;
  int M, K, Nout;
  int splits;           // K shares; split s runs slabs [s nk / splits, (s+1) nk / splits)
  // logits epilogue (LM head): bf16 output and per-row tile statistics
  uint16_t* yb;         // [M][ldy] bf16 bits
  long ldy;
  float2* tstats;       // [M][tiles_n] (max, sum exp(l - max)) of the tile's columns
  int tiles_n;
  int yb_vec;           // rows of yb start 16-byte aligned: store them 16 bytes at a time
  // few rows, gated, one launch: the first nu_blocks workgroups compute U's
  // split-K partials (A [r][K] into u_out) and count themselves in on
  // u_ctr[0]; the others wait for that count before their epilogue
  int nu_blocks;        // 0: U comes from an earlier launch
  const uint16_t* a;    // [r][K]
  float* u_out;         // = u, written by this launch
  int* u_ctr;           // [2] zero between calls: U workgroups done, output workgroups done
};

// Device-coherent (agent-scope) accesses for values one workgroup of a
// launch writes and another reads: they reach the point of coherence of the
// 8 XCDs instead of staying in the writer's L2.
__device__ __forceinline__ void store_f32_coherent(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_f4_coherent(const float* src) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(src));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float(static_cast<uint32_t>(a)), __uint_as_float(static_cast<uint32_t>(a >> 32)),
               __uint_as_float(static_cast<uint32_t>(b)), __uint_as_float(static_cast<uint32_t>(b >> 32))};
}
constexpr int kUSpinLimit = 1 << 22;  // polls of the U count before giving up

// One output element, fp32 or rounded to bf16 (nearest even).
__device__ __forceinline__ void store_y(void* y, bool ybf16, long i, float v) {
  if (ybf16) static_cast<uint16_t*>(y)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  else static_cast<float*>(y)[i] = v;
}
__device__ __forceinline__ float load_y(const void* y, bool ybf16, long i) {
  return ybf16 ? bf16_lo(static_cast<const uint16_t*>(y)[i]) : static_cast<const float*>(y)[i];
}

// Wait until at most n vector-memory operations of this wave are in flight
// and all of its LDS operations are done (exp counter not waited on).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// would wait for every direct load in flight); the waits the loop needs are
// explicit, and the empty asm keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes
// land at dst + 16 i (dst is the same for the whole wave).
__device__ __forceinline__ void load_lds16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Four waves in a 2 x 2 grid, each computing TM x TN blocks of 32 x 32, so
// a workgroup tile is 64 TM x 64 TN. Per 16-deep step a wave reads TM + TN
// operand fragments (1 KB each) from LDS for TM * TN MFMAs: larger wave tiles
// need less LDS bandwidth per MFMA, which is what bounds this loop.
template <int TM, int TN, int STAGES, int R16, bool kLogits = false>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmParams p) {
  constexpr int WM = 32 * TM, WN = 32 * TN;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int A_LOADS = BM / 32, B_LOADS = BN / 32;  // 1 KB direct loads per wave and slab
  constexpr int STAGE = (BM + BN) * kBK;                // elements per stage
  // one LDS object per stage, so the compiler can tell that reading a stage
  // does not wait for the direct loads into the others
  static_assert(STAGES >= 3 && STAGES <= kMaxStages, "stage count");
  static_assert(STAGES * STAGE * 2 <= kLdsBytes, "stages fit the LDS");
#define ISD_STAGE(i) __shared__ __attribute__((aligned(16))) uint16_t st##i[STAGES > i ? STAGE : 8];
  ISD_STAGE(0) ISD_STAGE(1) ISD_STAGE(2) ISD_STAGE(3) ISD_STAGE(4) ISD_STAGE(5)
#undef ISD_STAGE
  // (stages past STAGES are never named, so they take no LDS)
  auto stage_ptr = [&](int stage) -> uint16_t* {
    switch (stage) {
#define ISD_CASE(i) \
  case i:           \
    if constexpr (STAGES > i) return st##i;
      ISD_CASE(1) ISD_CASE(2) ISD_CASE(3) ISD_CASE(4) ISD_CASE(5)
#undef ISD_CASE
      default: return st0;
    }
  };

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int lane32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  // Workgroups reach the XCDs round robin (workgroup id mod 8). Each XCD
  // gets one contiguous run of tiles, M fastest, so a column block of W is
  // fetched into a single XCD's L2 and read from HBM about once.
  int m_blk, n_blk, split;
  {
    const int T = gridDim.x, nY = (p.M + BM - 1) / BM;
    const int q = T / kXcds, rem = T % kXcds;
    const int xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    const int t = xcd < rem ? xcd * (q + 1) + k : rem * (q + 1) + (xcd - rem) * q + k;
    const int tiles = T / p.splits;
    split = t / tiles;
    m_blk = (t % tiles % nY) * BM;
    n_blk = (t % tiles / nY) * BN;
  }

  // Slabs go from global memory straight into LDS (16-byte direct loads, no
  // register staging). A stage holds the slab's BM rows of x, then its BN rows
  // of W, 128 bytes per row with the 16-byte chunks XOR-swizzled: chunk c of
  // row r sits at slot c ^ (r % 8) ^ ((r / 8) % 2). The loads (lane i of a
  // load fills slot i % 8 of row i / 8 of an 8-row group) and the MFMA
  // operand reads (sixteen rows at one chunk, which land in both halves of
  // a 64-bank LDS line pair) then touch every bank once. Rows past the end
  // read the last valid row: output row i depends only on A row i and column
  // j only on B row j, and such rows and columns are never written.
  const int g_row = lane >> 3;
  auto g_chunk = [&](int group) { return (lane & 7) ^ g_row ^ (group & 1); };  // group = 8-row group index
  const uint16_t* a_src[A_LOADS];
  const uint16_t* b_src[B_LOADS];
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q)
    a_src[q] = p.x + static_cast<long>(min(m_blk + 8 * (wave + 4 * q) + g_row, p.M - 1)) * p.K + 8 * g_chunk(wave + 4 * q);
#pragma unroll
  for (int q = 0; q < B_LOADS; ++q)
    b_src[q] = p.w + static_cast<long>(min(n_blk + 8 * (wave + 4 * q) + g_row, p.Nout - 1)) * p.K + 8 * g_chunk(wave + 4 * q);
  auto load_slab = [&](int k0, int stage) {
    uint16_t* base = stage_ptr(stage);
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q)
      load_lds16(a_src[q] + k0, base + 8 * (wave + 4 * q) * kBK);
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q)
      load_lds16(b_src[q] + k0, base + (BM + 8 * (wave + 4 * q)) * kBK);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int sw = (lane32 & 7) ^ ((lane32 >> 3) & 1);  // swizzle of every operand row this lane reads
  // The operand fragments of step s+1 are read while step s multiplies.
  auto compute = [&](int stage) {
    const uint16_t* sA = stage_ptr(stage);
    const uint16_t* sB = sA + BM * kBK;
    constexpr int kSteps = kBK / 16;
    bf16x8 a[kSteps][TM], b[kSteps][TN];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int slot = ((2 * s + hh) ^ sw) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[s][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sA[(wm + 32 * i + lane32) * kBK + slot]));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[s][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sB[(wn + 32 * j + lane32) * kBK + slot]));
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
    // Software pipeline: the reads of step s+1 are issued right after the
    // MFMAs of step s (the scheduler would otherwise wait on LDS before
    // every step).
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
    for (int s = 0; s + 1 < kSteps; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
  };

  // STAGES-1 slabs in flight ahead of the one being multiplied. Slabs past
  // the last are clamped to it: their loads are harmless repeats into a stage
  // that is never read again.
  const int nk_all = p.K / kBK;
  const int kb = split * nk_all / p.splits, nk = (split + 1) * nk_all / p.splits - kb;
  constexpr int kLoads = A_LOADS + B_LOADS;

  // Gated: the U partials of the workgroup's rows and the B fragments of the
  // wave's column blocks are fetched ahead of the K loop, so the epilogue
  // waits on no memory. Thread t owns float4 t, t + 256, ... of the BM x r
  // U block; the partials are summed in split order (the order of the
  // stand-alone reduction kernel).
  // (Tiles whose U block and B fragments would not fit the register file,
  // 128-row tiles and the widest ranks, fetch them in the epilogue instead.)
  constexpr int kR16 = R16 > 0 ? R16 : 1;
  constexpr int r4 = 4 * kR16;  // float4 per U row
  constexpr int kUPer = (BM * r4) / 256;
  static_assert(R16 == 0 || (BM * r4) % 256 == 0, "U block split evenly over the threads");
  constexpr bool kPrefetch = R16 > 0 && TM == 1 && TN * R16 <= 18;
  f32x4 upart[kPrefetch ? kUPer : 1][kPrefetch ? kMaxSplits : 1];
  BFrag<kR16> bfr[kPrefetch ? TN : 1];
  if constexpr (kPrefetch) {
    const long pstride = static_cast<long>(p.M) * 16 * R16;  // elements between split partials
#pragma unroll
    for (int i = 0; i < kUPer; ++i) {
      const int e = tid + 256 * i, row = e / r4, q = e % r4;
      const float* src = p.u + static_cast<long>(min(m_blk + row, p.M - 1)) * 16 * R16 + 4 * q;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)  // missing splits re-read split 0, unused
        upart[i][sp] = *reinterpret_cast<const f32x4*>(src + (sp < p.u_splits ? sp : 0) * pstride);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = b_frag<R16>(p.b, p.Nout, n_blk + wn + 32 * j, lane32, hh);
  }
#pragma unroll
  for (int d = 0; d < STAGES - 1; ++d) load_slab((kb + min(d, nk - 1)) * kBK, d);
  f32x4 usum[kPrefetch ? kUPer : 1];
  if constexpr (kPrefetch) {
#pragma unroll
    for (int i = 0; i < kUPer; ++i) {
      f32x4 v = upart[i][0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplits; ++sp)
        if (sp < p.u_splits)
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = v[c] + upart[i][sp][c];
      usum[i] = v;
    }
  }
  // unrolled over kUnroll slabs: the compiler proves that reading one stage
  // need not wait for the loads into the others only inside one trip of the
  // loop, and waits for every load once per trip
  constexpr int kUnroll = STAGES * ((16 + STAGES - 1) / STAGES);
  for (int kt0 = 0; kt0 < nk; kt0 += kUnroll) {
#pragma unroll
    for (int dd = 0; dd < kUnroll; ++dd) {
      const int d = dd % STAGES;
      const int kt = kt0 + dd;
      if (kt >= nk) break;
      // this wave's loads of slab kt are done once only the STAGES-2 later
      // slabs' loads may still be in flight, and its reads of slab kt-1's
      // stage are done once no LDS operation is; after the barrier every
      // wave's part of slab kt is in LDS and nobody reads the stage that the
      // next load overwrites (slab kt-1's)
      wait_vm_lgkm0<(STAGES - 2) * kLoads>();
      stage_barrier();
      load_slab((kb + min(kt + STAGES - 1, nk - 1)) * kBK, (d + STAGES - 1) % STAGES);
      compute(d);
    }
  }
  wait_vm_lgkm0<0>();

  // LM head: the logits are rounded to bf16 (the values the accept step
  // reads) and parked in LDS as the tile's [BM][BN] rows (in stage 0, and
  // in stage 1 for the rows that do not fit a stage). Each thread then
  // takes 8 consecutive columns of a row: it stores them with one 16-byte
  // store (whole cache lines per row), and the 16 threads of a row form the
  // row's (max, sum of exp(l - max)) over the tile's 128 columns with a
  // fixed 4-step butterfly. Columns past Nout count as -inf.
  if constexpr (kLogits) {
    static_assert(R16 == 0, "the logits epilogue has no adapter");
    constexpr int kRowsPerStage = STAGE / BN;
    static_assert(BN == 128 && BM <= 2 * kRowsPerStage, "a 128-column tile fits two stages");
    uint16_t* const tile0 = stage_ptr(0);
    uint16_t* const tile1 = stage_ptr(1);
    auto tile_row = [&](int r) { return r < kRowsPerStage ? tile0 + r * BN : tile1 + (r - kRowsPerStage) * BN; };
    stage_barrier();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          tile_row(wm + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3))[wn + 32 * j + lane32] =
              static_cast<uint16_t>(f32_to_bf16_bits(acc[i][j][e]));
    wait_vm_lgkm0<0>();
    stage_barrier();
    for (int idx = tid; idx < BM * (BN / 8); idx += 256) {  // 16 threads (lanes 16q .. 16q+15) per row
      const int r = idx / (BN / 8), c = 8 * (idx % (BN / 8));
      const int row = m_blk + r, col = n_blk + c;
      const u32x4 v = *reinterpret_cast<const u32x4*>(tile_row(r) + c);
      if (row < p.M) {
        uint16_t* dst = p.yb + static_cast<long>(row) * p.ldy + col;
        if (p.yb_vec && col + 8 <= p.Nout) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const uint16_t* ev = reinterpret_cast<const uint16_t*>(&v);
          for (int k = 0; k < 8; ++k)
            if (col + k < p.Nout) dst[k] = ev[k];
        }
      }
      float x[8];
      unpack16(v, x);
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = col + k < p.Nout ? x[k] : -INFINITY;
        m = fmaxf(m, x[k]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, shfl_xor_f(m, off));
      float sum = 0.f;
      if (m != -INFINITY) {
        const float ml = m * kLog2e;
#pragma unroll
        for (int k = 0; k < 8; ++k) sum += weight_of(x[k], ml);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sum += shfl_xor_f(sum, off);
      if (c == 0 && row < p.M) p.tstats[static_cast<long>(row) * p.tiles_n + n_blk / BN] = make_float2(m, sum);
    }
    return;
  }

  // Gated: the workgroup writes the U rows of its BM rows into LDS, reusing
  // the stages (rows padded by 4 floats so the fragment reads spread over the
  // banks); each wave then splits its rows once for all of its column blocks.
  constexpr int kUStride = 16 * R16 + 4;
  constexpr int kURowsPerStage = R16 > 0 ? (STAGE * 2) / (kUStride * 4) : 1;
  static_assert(R16 == 0 || (BM + kURowsPerStage - 1) / kURowsPerStage <= STAGES, "U cache fits the stages");
  auto urow = [&](int row) -> float* {
    return reinterpret_cast<float*>(stage_ptr(row / kURowsPerStage)) + (row % kURowsPerStage) * kUStride;
  };
  if constexpr (R16 > 0) {
    stage_barrier();  // every wave is done with the stages
    if constexpr (kPrefetch) {
#pragma unroll
      for (int i = 0; i < kUPer; ++i) {
        const int e = tid + 256 * i, row = e / r4, q = e % r4;
        *reinterpret_cast<f32x4*>(urow(row) + 4 * q) = usum[i];
      }
    } else {
      const long pstride = static_cast<long>(p.M) * 16 * R16;
      for (int e = tid; e < BM * r4; e += 256) {
        const int row = e / r4, q = e % r4;
        const float* src = p.u + static_cast<long>(min(m_blk + row, p.M - 1)) * 16 * R16 + 4 * q;
        f32x4 part[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
          part[sp] = *reinterpret_cast<const f32x4*>(src + (sp < p.u_splits ? sp : 0) * pstride);
        f32x4 v = part[0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp)
          if (sp < p.u_splits)
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = v[c] + part[sp][c];
        *reinterpret_cast<f32x4*>(urow(row) + 4 * q) = v;
      }
    }
    wait_vm_lgkm0<0>();
    stage_barrier();
  }

  // Epilogue: register e of lane (j, hh) is row 8(e/4) + 4hh + e%4 of the
  // 32x32 block, column j. Gated: a MASK row takes acc + scale * delta, a
  // clean row takes acc itself.
  void* const y = p.ybf16 ? static_cast<void*>(static_cast<uint16_t*>(p.y) + static_cast<long>(split) * p.M * p.Nout)
                           : static_cast<void*>(static_cast<float*>(p.y) + static_cast<long>(split) * p.M * p.Nout);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m0 = m_blk + wm + 32 * i;
    int live = 0;
    UFrag<(R16 > 0 ? R16 : 1)> uf;
    if constexpr (R16 > 0) {
      const int mine = m0 + lane32 < p.M ? p.mask[m0 + lane32] != 0 : 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) live |= __shfl(mine, 8 * (e >> 2) + 4 * hh + (e & 3)) << e;
      if (__any(live)) uf = u_frag<R16>(urow(wm + 32 * i + lane32), hh);  // rows past M: never stored
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n0 = n_blk + wn + 32 * j;
      const int col = n0 + lane32;
      f32x16 dl = {};
      if constexpr (R16 > 0) {
        if (__any(live)) {
          if constexpr (kPrefetch) dl = lora_delta<R16>(uf, bfr[j]);
          else dl = lora_delta<R16>(uf, b_frag<R16>(p.b, p.Nout, n0, lane32, hh));
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (row < p.M && col < p.Nout)
          store_y(y, p.ybf16, static_cast<long>(row) * p.Nout + col,
                  ((live >> e) & 1) ? fmaf(p.scale, dl[e], acc[i][j][e]) : acc[i][j][e]);
      }
    }
  }
}

// Few rows (M <= 32: one sequence's stride block, or a handful): the tiled
// kernel would give Nout / 64 .. Nout / 192 workgroups, far fewer than CUs,
// each streaming its W columns with a few slabs in flight. Here one wave,
// as a workgroup of its own, owns one 32-column block of the output over
// the whole of K (Nout / 32 workgroups) and keeps S slabs in flight, as
// many as the wave's vector-memory counter tracks. A slab is the x rows
// (AL direct loads of 8 rows) and the block's 32 W rows (four loads), in
// the tiled kernel's swizzled LDS layout. Each 32x32 output block runs the
// tiled kernel's MFMA sequence, the same instruction on the same operands
// slab by slab in ascending K, and the gated epilogue is the tiled
// kernel's: every output has the bits the tiled kernel gives it. A split-K
// launch (U = x A^T's partials, at any M: one wave per 32x32 block and
// split, blockIdx.z the 32-row block) runs each split's share of the
// slabs, as the tiled kernel does.
template <int AL>
struct SkinnyShape {
  static constexpr int kLoads = AL + 4;  // 1 KB direct loads per slab
  static constexpr int S = 1 + 63 / kLoads < 12 ? 1 + 63 / kLoads : 12;  // slabs in flight + the one multiplied
  static constexpr int kARows = 8 * AL;
  static constexpr int STAGE = (kARows + 32) * kBK;  // elements
};

template <int AL, int R16>
__global__ __launch_bounds__(64) void gemm_skinny_kernel(GemmParams p) {
  using SK = SkinnyShape<AL>;
  constexpr int S = SK::S, STAGE = SK::STAGE, kARows = SK::kARows, kLoads = SK::kLoads;
  static_assert(S >= 3 && S <= 12, "stage count");
  static_assert((S - 2) * kLoads < 64, "loads in flight fit the counter");
  // one LDS object per stage, as in the tiled kernel
#define ISD_SK_STAGE(i) __shared__ __attribute__((aligned(16))) uint16_t sk##i[S > i ? STAGE : 8];
  ISD_SK_STAGE(0) ISD_SK_STAGE(1) ISD_SK_STAGE(2) ISD_SK_STAGE(3) ISD_SK_STAGE(4) ISD_SK_STAGE(5)
  ISD_SK_STAGE(6) ISD_SK_STAGE(7) ISD_SK_STAGE(8) ISD_SK_STAGE(9) ISD_SK_STAGE(10) ISD_SK_STAGE(11)
#undef ISD_SK_STAGE
  auto stage_ptr = [&](int stage) -> uint16_t* {
    switch (stage) {
#define ISD_CASE(i) \
  case i:           \
    if constexpr (S > i) return sk##i;
      ISD_CASE(1) ISD_CASE(2) ISD_CASE(3) ISD_CASE(4) ISD_CASE(5) ISD_CASE(6) ISD_CASE(7) ISD_CASE(8) ISD_CASE(9)
      ISD_CASE(10) ISD_CASE(11)
#undef ISD_CASE
      default: return sk0;
    }
  };
  constexpr int kR16 = R16 > 0 ? R16 : 1;
  constexpr int kUStride = 16 * R16 + 4;  // U rows in LDS, padded as in the tiled kernel
  __shared__ __attribute__((aligned(16))) float s_u[R16 > 0 ? kARows * kUStride : 4];

  const int lane = threadIdx.x, lane32 = lane & 31, hh = lane >> 5;
  // In a gated launch that also computes U (p.nu_blocks > 0), workgroup i <
  // nu_blocks is U's split-K partial of rank columns 32 (i % ub) .. and split
  // i / ub, exactly as the ungated partial launch computes it; the others
  // are the output blocks.
  constexpr int kRank = 16 * (R16 > 0 ? R16 : 1);
  constexpr int kUb = (kRank + 31) / 32;  // 32-column blocks of U
  const bool u_role = R16 > 0 && static_cast<int>(blockIdx.x) < p.nu_blocks;
  const int yblk = static_cast<int>(blockIdx.x) - p.nu_blocks;
  const uint16_t* const wmat = u_role ? p.a : p.w;
  const int nout = u_role ? kRank : p.Nout;
  const int n0 = u_role ? (static_cast<int>(blockIdx.x) % kUb) * 32 : (R16 > 0 ? yblk : static_cast<int>(blockIdx.x)) * 32;
  // rows m0 .. m0+31 (blockIdx.z > 0 only for the ungated split-K partials;
  // the gated epilogue runs with M <= 32, one row block)
  const int m0 = blockIdx.z * 32;
  // Load q of a slab fills 8 LDS rows, lane i row i / 8 at slot i % 8,
  // with the chunk the swizzle puts there (chunk c of row r sits at slot
  // c ^ (r % 8) ^ ((r / 8) % 2)). x rows past M read row M - 1 and W rows
  // past Nout row Nout - 1: such rows and columns are never stored.
  const int g_row = lane >> 3;
  const uint16_t* a_src[AL];
  const uint16_t* b_src[4];
#pragma unroll
  for (int q = 0; q < AL; ++q)
    a_src[q] = p.x + static_cast<long>(min(m0 + 8 * q + g_row, p.M - 1)) * p.K + 8 * ((lane & 7) ^ g_row ^ (q & 1));
#pragma unroll
  for (int q = 0; q < 4; ++q)
    b_src[q] = wmat + static_cast<long>(min(n0 + 8 * q + g_row, nout - 1)) * p.K + 8 * ((lane & 7) ^ g_row ^ (q & 1));
  auto load_slab = [&](int k0, int stage) {
    uint16_t* base = stage_ptr(stage);
#pragma unroll
    for (int q = 0; q < AL; ++q) load_lds16(a_src[q] + k0, base + 8 * q * kBK);
#pragma unroll
    for (int q = 0; q < 4; ++q) load_lds16(b_src[q] + k0, base + (kARows + 8 * q) * kBK);
  };

  // Operand rows of this lane: W row lane32 of the block, x row lane32
  // (lanes past the staged x rows read a staged row; their output rows are
  // at or past M).
  const int ra = lane32 & (kARows - 1);
  const int swa = (ra & 7) ^ ((ra >> 3) & 1), swb = (lane32 & 7) ^ ((lane32 >> 3) & 1);
  f32x16 acc = {};
  auto compute = [&](int stage) {
    const uint16_t* sA = stage_ptr(stage);
    const uint16_t* sB = sA + kARows * kBK;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sA[ra * kBK + ((2 * s + hh) ^ swa) * 8]));
      b[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sB[lane32 * kBK + ((2 * s + hh) ^ swb) * 8]));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
  };

  // split-K (U's partials): split blockIdx.y runs the tiled kernel's share
  // of the slabs, [s nk / splits, (s+1) nk / splits), into its own output
  const int split = u_role ? static_cast<int>(blockIdx.x) / kUb : static_cast<int>(blockIdx.y);
  const int splits = u_role ? p.u_splits : p.splits;
  const int nk_all = p.K / kBK;
  const int kb = split * nk_all / splits, nk = (split + 1) * nk_all / splits - kb;
#pragma unroll
  for (int d = 0; d < S - 1; ++d) load_slab((kb + min(d, nk - 1)) * kBK, d);

  // Gated: the U rows (split-K partials summed in split order, as the tiled
  // kernel sums them) go to LDS, the B fragments and mask bits to registers.
  // With U from an earlier launch the rows are staged while the first slabs
  // are in flight; with U computed in this launch, after the K loop, once
  // every U workgroup has counted itself in.
  auto stage_u = [&](bool coherent) {
    if constexpr (R16 > 0) {
      constexpr int r4 = 4 * R16;
      const long pstride = static_cast<long>(p.M) * 16 * R16;
      for (int e = lane; e < p.M * r4; e += 64) {
        const int row = e / r4, q = e % r4;
        const float* src = p.u + static_cast<long>(row) * 16 * R16 + 4 * q;
        f32x4 part[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) {
          const float* ps = src + (sp < p.u_splits ? sp : 0) * pstride;
          part[sp] = coherent ? load_f4_coherent(ps) : *reinterpret_cast<const f32x4*>(ps);
        }
        f32x4 v = part[0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp)
          if (sp < p.u_splits)
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = v[c] + part[sp][c];
        *reinterpret_cast<f32x4*>(&s_u[row * kUStride + 4 * q]) = v;
      }
    }
  };
  int mine = 0;
  BFrag<kR16> bfr;
  if constexpr (R16 > 0) {
    if (!u_role) {
      if (p.nu_blocks == 0) stage_u(false);
      bfr = b_frag<R16>(p.b, p.Nout, n0, lane32, hh);
      mine = lane32 < p.M ? p.mask[lane32] != 0 : 0;
    }
  }

  // unrolled over S slabs, so every stage index is a constant (as in the
  // tiled kernel); one wave, so the waits alone order the stages
  for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
    for (int d = 0; d < S; ++d) {
      const int kt = kt0 + d;
      if (kt >= nk) break;
      // slab kt has landed once only the S-2 later slabs' loads may be in
      // flight, and the reads of slab kt-1's stage (the one the next load
      // overwrites) are done once no LDS operation is
      wait_vm_lgkm0<(S - 2) * kLoads>();
      load_slab((kb + min(kt + S - 1, nk - 1)) * kBK, (d + S - 1) % S);
      compute(d);
    }
  }
  wait_vm_lgkm0<0>();

  if constexpr (R16 > 0) {
    if (u_role) {
      // U's partial of this split: stored device-coherently, completed,
      // then counted in (no reply needed)
      const int col = n0 + lane32;
      float* const dst = p.u_out + static_cast<long>(split) * p.M * kRank;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * hh + (e & 3);
        if (row < p.M && col < kRank) store_f32_coherent(dst + static_cast<long>(row) * kRank + col, acc[e]);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      if (lane == 0) __hip_atomic_fetch_add(&p.u_ctr[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  // U computed in this launch: wait (lane 0, bounded) until every U
  // workgroup has counted itself in, stage the rows, then count this
  // workgroup in; the last output workgroup returns both counts to zero.
  // Every workgroup of such a launch fits on the GPU at once (the host
  // checks), so the U workgroups always run; should the wait still reach
  // its bound, the MASK rows of this block come out NaN.
  bool u_ok = true;
  if constexpr (R16 > 0) {
    if (p.nu_blocks > 0) {
      int ok = 1;
      if (lane == 0) {
        int spins = 0;
        while (__hip_atomic_load(&p.u_ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < p.nu_blocks) {
          if (++spins > kUSpinLimit) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      asm volatile("" ::: "memory");
      u_ok = __shfl(ok, 0) != 0;
      if (u_ok) stage_u(true);
      wait_vm_lgkm0<0>();
      if (lane == 0) {
        const int ny = static_cast<int>(gridDim.x) - p.nu_blocks;
        if (__hip_atomic_fetch_add(&p.u_ctr[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ny - 1) {
          __hip_atomic_fetch_add(&p.u_ctr[0], -p.nu_blocks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&p.u_ctr[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // Epilogue (the tiled kernel's): register e of lane (j, hh) is row
  // 8(e/4) + 4hh + e%4, column j; a MASK row takes acc + scale * delta.
  int live = 0;
  f32x16 dl = {};
  if constexpr (R16 > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) live |= __shfl(mine, 8 * (e >> 2) + 4 * hh + (e & 3)) << e;
    if (__any(live)) {
      if (u_ok)
        dl = lora_delta<R16>(u_frag<R16>(lane32 < p.M ? &s_u[lane32 * kUStride] : nullptr, hh), bfr);
      else
#pragma unroll
        for (int e = 0; e < 16; ++e) dl[e] = NAN;
    }
  }
  const int col = n0 + lane32;
  void* const y = p.ybf16 ? static_cast<void*>(static_cast<uint16_t*>(p.y) + static_cast<long>(split) * p.M * p.Nout)
                           : static_cast<void*>(static_cast<float*>(p.y) + static_cast<long>(split) * p.M * p.Nout);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
    if (row < p.M && col < p.Nout)
      store_y(y, p.ybf16, static_cast<long>(row) * p.Nout + col,
              ((live >> e) & 1) ? fmaf(p.scale, dl[e], acc[e]) : acc[e]);
  }
}

// y[m] += scale * (U B^T)[m] on MASK rows only, one wave per 32x32 tile of
// y; tiles without a MASK row are skipped and clean rows are never written.
// The delta is the GEMM epilogue's, instruction for instruction.
struct DeltaParams {
  const float* u;      // [M][r]
  const uint16_t* b;   // [Nout][r]
  const uint8_t* mask; // [M]
  void* y;             // [M][Nout], fp32 or bf16 bits
  int ybf16;
  int M, Nout;
  float scale;
};

template <int R16>
__global__ __launch_bounds__(256) void lora_delta_kernel(DeltaParams p) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lane32 = lane & 31, hh = lane >> 5;
  const int tiles_n = (p.Nout + 31) / 32;
  const long tile = static_cast<long>(blockIdx.x) * 4 + wave;
  if (tile >= static_cast<long>((p.M + 31) / 32) * tiles_n) return;
  const int m0 = static_cast<int>(tile / tiles_n) * 32, n0 = static_cast<int>(tile % tiles_n) * 32;
  const int bcol = n0 + lane32;
  const int mine = m0 + lane32 < p.M ? p.mask[m0 + lane32] != 0 : 0;
  int live = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) live |= (__shfl(mine, 8 * (e >> 2) + 4 * hh + (e & 3)) && bcol < p.Nout) << e;
  if (!__any(live)) return;
  // y of the MASK rows is loaded before the delta's operands arrive
  float yv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
    yv[e] = ((live >> e) & 1) ? load_y(p.y, p.ybf16, static_cast<long>(row) * p.Nout + bcol) : 0.f;
  }
  const UFrag<R16> uf = u_frag<R16>(m0 + lane32 < p.M ? p.u + static_cast<long>(m0 + lane32) * 16 * R16 : nullptr, hh);
  const f32x16 dl = lora_delta<R16>(uf, b_frag<R16>(p.b, p.Nout, n0, lane32, hh));
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if ((live >> e) & 1) {
      const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
      store_y(p.y, p.ybf16, static_cast<long>(row) * p.Nout + bcol, fmaf(p.scale, dl[e], yv[e]));
    }
  }
}

// U = sum of the split-K partials of x A^T, in split order.
__global__ __launch_bounds__(256) void lora_u_reduce_kernel(const float* part, float* U, long n, int splits) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int k = 1; k < splits; ++k) s += part[static_cast<long>(k) * n + i];
  U[i] = s;
}

}  // namespace isd

// ================================================================ host API
namespace {
using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Tile choice depends only on (M, Nout) and the CU count, never on the
// data, and every choice gives each output the same reduction order. A CU
// streams its workgroups' operand slabs at a rate of its own that the chip
// seldom saturates (the weights come from HBM, the rows of x from L2), so
// the choice minimises the bytes of the busiest CU, rounds of workgroups
// per CU x (BM + BN) rows per slab; on a tie the earlier (larger) tile wins
// (fewer LDS bytes per MFMA). The large tiles run one workgroup per CU with
// four stages; 64 x 64 tiles take five (two workgroups per CU), or three
// for the split-K partials of U.
template <int TM, int TN, int STAGES, int R16, bool kLogits = false>
hipError_t launch_tile(const GemmParams& p, hipStream_t stream) {
  const long tiles = static_cast<long>((p.M + 64 * TM - 1) / (64 * TM)) * ((p.Nout + 64 * TN - 1) / (64 * TN));
  hipLaunchKernelGGL((gemm_nt_kernel<TM, TN, STAGES, R16, kLogits>), dim3(static_cast<unsigned>(tiles * p.splits)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int R16>
hipError_t launch_gemm_r(const GemmParams& p, hipStream_t stream) {
  const long cus = isd_device_cus_internal();
  constexpr int kShapes[5][2] = {{2, 3}, {1, 3}, {2, 2}, {1, 2}, {1, 1}};
  int pick = 4;
  long best = -1;
  for (int i = p.splits == 1 ? 0 : 4; i < 5; ++i) {
    const int tm = kShapes[i][0], tn = kShapes[i][1];
    const long wgs = static_cast<long>((p.M + 64 * tm - 1) / (64 * tm)) * ((p.Nout + 64 * tn - 1) / (64 * tn)) * p.splits;
    const long cost = (wgs + cus - 1) / cus * (64 * tm + 64 * tn);
    if (best < 0 || cost < best) {
      best = cost;
      pick = i;
    }
  }
  // Few rows: one wave per 32 output columns (and split). The ungated
  // split-K partials of U run here at any M, one wave per 32 x 32 output
  // block and split: each wave keeps all of its split's slabs in flight.
  if (p.M <= 32 || (R16 == 0 && p.splits > 1)) {
    const unsigned mblocks = R16 == 0 ? static_cast<unsigned>((p.M + 31) / 32) : 1u;
    // (with p.nu_blocks > 0 the U workgroups come first in x)
    const dim3 grid(static_cast<unsigned>(p.nu_blocks + (p.Nout + 31) / 32), static_cast<unsigned>(p.splits), mblocks);
    if (mblocks > 1) hipLaunchKernelGGL((gemm_skinny_kernel<4, R16>), grid, dim3(64), 0, stream, p);
    else if (p.M <= 8) hipLaunchKernelGGL((gemm_skinny_kernel<1, R16>), grid, dim3(64), 0, stream, p);
    else if (p.M <= 16) hipLaunchKernelGGL((gemm_skinny_kernel<2, R16>), grid, dim3(64), 0, stream, p);
    else hipLaunchKernelGGL((gemm_skinny_kernel<4, R16>), grid, dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  switch (pick) {
    case 0: return launch_tile<2, 3, 3, R16>(p, stream);
    case 1: return launch_tile<1, 3, 4, R16>(p, stream);
    case 2: return launch_tile<2, 2, 4, R16>(p, stream);
    case 3: return launch_tile<1, 2, 4, R16>(p, stream);
    default: return launch_tile<1, 1, 5, R16>(p, stream);
  }
}

// Chunk statistics of the logits from the tile statistics: one wave per
// (row, chunk); lane k holds tile k of the chunk (the 64 tiles of 128
// columns that make 8192 entries) and a fixed butterfly merges them, so
// lane 0's result depends only on the row's tiles.
__global__ __launch_bounds__(256) void logits_chunk_stats_kernel(const float2* tstats, int tiles_n, int M, int nch,
                                                                 float2* out) {
  static_assert(kVocabChunk / kLogitsTileN == kWave, "one tile per lane");
  const long item = static_cast<long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (item >= static_cast<long>(M) * nch) return;
  const int lane = threadIdx.x % kWave;
  const int m = static_cast<int>(item / nch), c = static_cast<int>(item % nch);
  const int k = c * kWave + lane;
  float mx = -INFINITY, sum = 0.f;
  if (k < tiles_n) {
    const float2 t = tstats[static_cast<long>(m) * tiles_n + k];
    mx = t.x;
    sum = t.y;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) merge_ms(mx, sum, __shfl_xor(mx, off, kWave), __shfl_xor(sum, off, kWave));
  if (lane == 0) out[item] = make_float2(mx, sum);
}

hipError_t launch_gemm(const GemmParams& p, int r, hipStream_t stream) {
  switch (r / 16) {
    case 0: return launch_gemm_r<0>(p, stream);
    case 1: return launch_gemm_r<1>(p, stream);
    case 2: return launch_gemm_r<2>(p, stream);
    case 3: return launch_gemm_r<3>(p, stream);
    case 4: return launch_gemm_r<4>(p, stream);
    case 5: return launch_gemm_r<5>(p, stream);
    case 6: return launch_gemm_r<6>(p, stream);
    case 7: return launch_gemm_r<7>(p, stream);
    default: return launch_gemm_r<8>(p, stream);
  }
}

// Split count of U = x A^T: a function of K only (so U's bits do not depend
// on M), the largest of 8, 4, 2, 1 that divides the slab count.
int u_splits(int K) {
  const int nk = K / kBK;
  int s = kMaxSplits;
  while (s > 1 && nk % s != 0) s /= 2;
  return s;
}

size_t part_bytes(int M, int r) { return (static_cast<size_t>(M) * r * sizeof(float) * kMaxSplits + 255) & ~static_cast<size_t>(255); }

// LoRA workspace: a counter pair (zero between calls) in its first 256
// bytes, then U's split-K partials, then U.
constexpr size_t kLoraCtrlBytes = 256;
float* lora_parts_of(void* ws) { return reinterpret_cast<float*>(static_cast<char*>(ws) + kLoraCtrlBytes); }

// Split-K partials of U = x A^T into the workspace.
hipError_t launch_lora_u_partials(const void* x, const void* A, int M, int K, int r, void* ws, hipStream_t stream) {
  GemmParams g{};
  g.x = static_cast<const uint16_t*>(x);
  g.w = static_cast<const uint16_t*>(A);
  g.y = lora_parts_of(ws);
  g.M = M;
  g.K = K;
  g.Nout = r;
  g.splits = u_splits(K);
  return launch_gemm_r<0>(g, stream);
}

// U = x A^T into the workspace: split-K partials, then their sum.
hipError_t launch_lora_u(const void* x, const void* A, int M, int K, int r, void* ws, hipStream_t stream) {
  hipError_t e = launch_lora_u_partials(x, A, M, K, r, ws, stream);
  if (e != hipSuccess) return e;
  float* U = reinterpret_cast<float*>(reinterpret_cast<char*>(lora_parts_of(ws)) + part_bytes(M, r));
  const long n = static_cast<long>(M) * r;
  hipLaunchKernelGGL(lora_u_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const float*>(lora_parts_of(ws)), U, n, u_splits(K));
  return hipGetLastError();
}

const float* lora_u_of(void* ws, int M, int r) {
  return reinterpret_cast<const float*>(reinterpret_cast<char*>(lora_parts_of(ws)) + part_bytes(M, r));
}

// Workgroups of gemm_skinny_kernel<AL, R16> the current GPU holds at once
// (its occupancy times its CUs), looked up once per device.
template <int AL, int R16>
long skinny_capacity() {
  static std::mutex mu;
  static long cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && cache[dev] > 0) return cache[dev];
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_skinny_kernel<AL, R16>, 64, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const long total = static_cast<long>(per_cu) * isd_device_cus_internal();
  if (dev >= 0) cache[dev] = total;
  return total;
}

hipError_t launch_delta(const float* U, const void* B, const uint8_t* mask, int M, int Nout, int r, float scale,
                        void* y, int ybf16, hipStream_t stream) {
  DeltaParams d{};
  d.u = U;
  d.b = static_cast<const uint16_t*>(B);
  d.mask = mask;
  d.y = y;
  d.ybf16 = ybf16;
  d.M = M;
  d.Nout = Nout;
  d.scale = scale;
  const long tiles = static_cast<long>((M + 31) / 32) * ((Nout + 31) / 32);
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
  switch (r / 16) {
    case 1: hipLaunchKernelGGL(lora_delta_kernel<1>, grid, dim3(256), 0, stream, d); break;
    case 2: hipLaunchKernelGGL(lora_delta_kernel<2>, grid, dim3(256), 0, stream, d); break;
    case 3: hipLaunchKernelGGL(lora_delta_kernel<3>, grid, dim3(256), 0, stream, d); break;
    case 4: hipLaunchKernelGGL(lora_delta_kernel<4>, grid, dim3(256), 0, stream, d); break;
    case 5: hipLaunchKernelGGL(lora_delta_kernel<5>, grid, dim3(256), 0, stream, d); break;
    case 6: hipLaunchKernelGGL(lora_delta_kernel<6>, grid, dim3(256), 0, stream, d); break;
    case 7: hipLaunchKernelGGL(lora_delta_kernel<7>, grid, dim3(256), 0, stream, d); break;
    default: hipLaunchKernelGGL(lora_delta_kernel<8>, grid, dim3(256), 0, stream, d); break;
  }
  return hipGetLastError();
}

// skinny_capacity for the kernel a gated call with M <= 32 rows and rank r
// launches (the row count picks AL as launch_gemm_r does).
template <int R16>
long skinny_capacity_r(int M) {
  return M <= 8 ? skinny_capacity<1, R16>() : (M <= 16 ? skinny_capacity<2, R16>() : skinny_capacity<4, R16>());
}
long skinny_capacity_of(int M, int r) {
  switch (r / 16) {
    case 1: return skinny_capacity_r<1>(M);
    case 2: return skinny_capacity_r<2>(M);
    case 3: return skinny_capacity_r<3>(M);
    case 4: return skinny_capacity_r<4>(M);
    case 5: return skinny_capacity_r<5>(M);
    case 6: return skinny_capacity_r<6>(M);
    case 7: return skinny_capacity_r<7>(M);
    default: return skinny_capacity_r<8>(M);
  }
}

int check_gemm_args(const void* x, const void* W, int M, int K, int Nout, const void* y, int ydtype) {
  if (M < 0 || K < 0 || Nout < 0) return ISD_E_INVALID;
  if (ydtype != ISD_F32 && ydtype != ISD_BF16) return ISD_E_UNSUPPORTED;
  if (M == 0 || Nout == 0) return ISD_OK;
  if (!x || !W || !y) return ISD_E_INVALID;
  if ((reinterpret_cast<uintptr_t>(y) & (ydtype == ISD_F32 ? 3u : 1u)) != 0) return ISD_E_INVALID;
  if (K == 0 || K % kBK != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W)) return ISD_E_INVALID;
  return ISD_OK;
}

int check_lora_args(const void* A, const void* B, const uint8_t* mask, int r, void* ws, size_t ws_bytes, int M) {
  if (!A || !B || !mask) return ISD_E_INVALID;
  if (r < 16 || r > 128 || r % 16 != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(A) || !aligned16(B)) return ISD_E_INVALID;
  if (!ws || ws_bytes < isd_lora_workspace_size(M, r) || !aligned16(ws)) return ISD_E_WORKSPACE;
  return ISD_OK;
}

}  // namespace

extern "C" {

int isd_linear(const void* x, const void* W, int M, int K, int Nout, void* y, int ydtype, hipStream_t stream) {
  int rc = check_gemm_args(x, W, M, K, Nout, y, ydtype);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(W);
  p.y = y;
  p.ybf16 = ydtype == ISD_BF16;
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  p.splits = 1;
  return launch_gemm(p, 0, stream) == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

size_t isd_lora_workspace_size(int M, int r) {
  if (M < 0 || r < 0) return 0;
  return kLoraCtrlBytes + part_bytes(M, r) + static_cast<size_t>(M) * r * sizeof(float);
}

int gated_lora_apply(const void* x, const void* A, const void* B, const uint8_t* is_mask, int M, int K, int Nout,
                     int r, float scale, void* y, int ydtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_args(x, A, M, K, Nout, y, ydtype);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  if (launch_lora_u(x, A, M, K, r, ws, stream) != hipSuccess) return ISD_E_LAUNCH;
  return launch_delta(lora_u_of(ws, M, r), B, is_mask, M, Nout, r, scale, y, ydtype == ISD_BF16, stream) == hipSuccess
             ? ISD_OK
             : ISD_E_LAUNCH;
}

int isd_linear_gated(const void* x, const void* W, const void* A, const void* B, const uint8_t* is_mask, int M, int K,
                     int Nout, int r, float scale, void* y, int ydtype, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int rc = check_gemm_args(x, W, M, K, Nout, y, ydtype);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  // U's split-K partials; the GEMM sums them (in split order, as the
  // reduction kernel of gated_lora_apply does) when it stages its U rows.
  // Few rows: U's workgroups join the GEMM's launch when all of its
  // workgroups fit on the GPU at once; otherwise U has a launch of its own.
  const int nu = (r + 31) / 32 * u_splits(K);
  const bool one_launch = M <= 32 && nu + (static_cast<long>(Nout) + 31) / 32 <= skinny_capacity_of(M, r);
  if (!one_launch && launch_lora_u_partials(x, A, M, K, r, ws, stream) != hipSuccess) return ISD_E_LAUNCH;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(W);
  p.y = y;
  p.ybf16 = ydtype == ISD_BF16;
  p.u = lora_parts_of(ws);
  p.u_splits = u_splits(K);
  if (one_launch) {
    p.nu_blocks = nu;
    p.a = static_cast<const uint16_t*>(A);
    p.u_out = lora_parts_of(ws);
    p.u_ctr = static_cast<int*>(ws);
  }
  p.b = static_cast<const uint16_t*>(B);
  p.mask = is_mask;
  p.scale = scale;
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  p.splits = 1;
  return launch_gemm(p, r, stream) == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

size_t isd_lm_head_workspace_size(int M, int V) {
  if (M < 0 || V < 1) return 0;
  return (static_cast<size_t>(M) * ((V + kLogitsTileN - 1) / kLogitsTileN) * sizeof(float2) + 255) &
         ~static_cast<size_t>(255);
}

int isd_lm_head(const void* h, const void* W, int M, int K, int V, void* logits, int64_t ld, float* chunk_stats,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || K < 0 || V < 1 || ld < V) return ISD_E_INVALID;
  if (M == 0) return ISD_OK;
  if (!h || !W || !logits || !chunk_stats) return ISD_E_INVALID;
  if (K == 0 || K % kBK != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(h) || !aligned16(W)) return ISD_E_INVALID;
  if (!ws || ws_bytes < isd_lm_head_workspace_size(M, V) || !aligned16(ws)) return ISD_E_WORKSPACE;
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(h);
  p.w = static_cast<const uint16_t*>(W);
  p.M = M;
  p.K = K;
  p.Nout = V;
  p.splits = 1;
  p.yb = static_cast<uint16_t*>(logits);
  p.ldy = static_cast<long>(ld);
  p.tstats = static_cast<float2*>(ws);
  p.tiles_n = (V + kLogitsTileN - 1) / kLogitsTileN;
  p.yb_vec = ld % 8 == 0 && aligned16(logits);
  // a tile of 128 columns and 256, 128 or 64 rows, by the same busiest-CU
  // rule as the projections (the earlier, taller tile wins a tie); the
  // 256-row tile has three stages of 48 KB, the others four of 32 or 24 KB
  const long cus = isd_device_cus_internal();
  auto cost = [&](int tm) {
    const long wgs = static_cast<long>((M + 64 * tm - 1) / (64 * tm)) * p.tiles_n;
    return (wgs + cus - 1) / cus * (64 * tm + kLogitsTileN);
  };
  const int tm = cost(4) <= cost(2) ? (cost(4) <= cost(1) ? 4 : 1) : (cost(2) <= cost(1) ? 2 : 1);
  hipError_t e = tm == 4   ? launch_tile<4, 2, 3, 0, true>(p, stream)
                 : tm == 2 ? launch_tile<2, 2, 4, 0, true>(p, stream)
                           : launch_tile<1, 2, 4, 0, true>(p, stream);
  if (e != hipSuccess) return ISD_E_LAUNCH;
  const int nch = (V + kVocabChunk - 1) / kVocabChunk;
  const long n = static_cast<long>(M) * nch;  // one wave each, four per workgroup
  hipLaunchKernelGGL(logits_chunk_stats_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const float2*>(ws), p.tiles_n, M, nch, reinterpret_cast<float2*>(chunk_stats));
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // extern "C"

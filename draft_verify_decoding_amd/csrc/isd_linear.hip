// Base projection GEMM and the gated LoRA of lossless R-ISD (gfx950).
//
// The adapter acts only at MASK positions so that clean positions keep the
// base model's outputs bit for bit (I-DLM, fr.news.hada.io, "Speedup Factor
// Explorer" and "Documentation et ressources > Lossless R-ISD"). Here that
// means: y = x W^T on every row with one fixed MFMA reduction order; MASK rows
// then get y += s * (x A^T) B^T and clean rows are never written again.
//
// GEMM: y[M][Nout] fp32 = x[M][K] bf16 . W[Nout][K]^T bf16 ("NT": both
// operands K-contiguous). Workgroup tile 2*WM x 2*WN (four waves, each WM x WN
// in 32x32 MFMA blocks), K in slabs of 64 through double-buffered LDS with
// padded rows (72 elements) so the 16-byte operand reads are conflict-free,
// several slabs in flight in a register ring. The per-output reduction order
// is slab by slab in ascending K and does not depend on M, the tile choice,
// the other rows or the mask.
// LoRA: U = x A^T comes out of the same GEMM as r extra output columns (A's
// rows appended to W's); delta = U B^T then runs on bf16 MFMA with U split
// into bf16 high and low halves (about 16 mantissa bits), and is added with
// one fma to MASK rows only.
#include "isd_common.hpp"

namespace isd {

constexpr int kBK = 64;
constexpr int kXcds = 8;  // XCDs of an MI355X
constexpr int kLdsStride = kBK + 8;  // elements per LDS row

struct GemmParams {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [Nout][K]
  const uint16_t* a;  // optional [r][K]: output columns Nout..Nout+r-1 use A's rows
  float* y;           // [M][Nout]
  float* u;           // [M][r] receives x A^T when a != nullptr
  int M, K, Nout, r;
};

template <int WM, int WN, int DEPTH>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmParams p) {
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_ROUNDS = BM * kBK / 8 / 256;  // 16-byte loads per thread
  constexpr int B_ROUNDS = BN * kBK / 8 / 256;
  static_assert(A_ROUNDS >= 1 && B_ROUNDS >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * kLdsStride];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int lane32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  // Workgroups reach the XCDs round robin (workgroup id mod 8). Each XCD
  // gets one contiguous run of tiles, M fastest, so a column block of W is
  // fetched into a single XCD's L2 and read from HBM about once.
  int m_blk, n_blk;
  {
    const int T = gridDim.x, nY = (p.M + BM - 1) / BM;
    const int q = T / kXcds, rem = T % kXcds;
    const int xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    const int t = xcd < rem ? xcd * (q + 1) + k : rem * (q + 1) + (xcd - rem) * q + k;
    m_blk = (t % nY) * BM;
    n_blk = (t / nY) * BN;
  }

  // Global->register staging: thread loads rows (tid / 8) + 32*q, 16 bytes at
  // column 8 * (tid % 8) of the 64-wide K slab. A ring of DEPTH register
  // sets keeps DEPTH slabs in flight; LDS is double-buffered. Every load is
  // unconditional (no divergent branch around it), so the compiler waits
  // only for the slab it is about to store: rows past the end read the last
  // valid row instead. Output row i depends only on A row i and column j only
  // on B row j, and such rows and columns are never written.
  const int ld_row = tid >> 3, ld_col = (tid & 7) * 8;
  const uint16_t* a_src[A_ROUNDS];
  const uint16_t* b_src[B_ROUNDS];
#pragma unroll
  for (int q = 0; q < A_ROUNDS; ++q)
    a_src[q] = p.x + static_cast<long>(min(m_blk + ld_row + 32 * q, p.M - 1)) * p.K + ld_col;
#pragma unroll
  for (int q = 0; q < B_ROUNDS; ++q) {
    const int row = min(n_blk + ld_row + 32 * q, p.Nout + p.r - 1);
    b_src[q] = (row < p.Nout ? p.w + static_cast<long>(row) * p.K : p.a + static_cast<long>(row - p.Nout) * p.K) +
               ld_col;
  }
  u32x4 ra[DEPTH][A_ROUNDS], rb[DEPTH][B_ROUNDS];
  auto load_slab = [&](int k0, u32x4 (&a)[A_ROUNDS], u32x4 (&b)[B_ROUNDS]) {
#pragma unroll
    for (int q = 0; q < A_ROUNDS; ++q) a[q] = *reinterpret_cast<const u32x4*>(a_src[q] + k0);
#pragma unroll
    for (int q = 0; q < B_ROUNDS; ++q) b[q] = *reinterpret_cast<const u32x4*>(b_src[q] + k0);
  };
  auto store_slab = [&](int buf, const u32x4 (&a)[A_ROUNDS], const u32x4 (&b)[B_ROUNDS]) {
#pragma unroll
    for (int q = 0; q < A_ROUNDS; ++q)
      *reinterpret_cast<u32x4*>(&sA[buf][(ld_row + 32 * q) * kLdsStride + ld_col]) = a[q];
#pragma unroll
    for (int q = 0; q < B_ROUNDS; ++q)
      *reinterpret_cast<u32x4*>(&sB[buf][(ld_row + 32 * q) * kLdsStride + ld_col]) = b[q];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&sA[buf][(wm + 32 * i + lane32) * kLdsStride + 16 * s + 8 * hh]));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&sB[buf][(wn + 32 * j + lane32) * kLdsStride + 16 * s + 8 * hh]));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Slabs past the last are clamped to it: their loads and the final LDS
  // store are harmless repeats whose data is never read.
  const int nk = p.K / kBK;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_slab(min(d, nk - 1) * kBK, ra[d], rb[d]);
  store_slab(0, ra[0], rb[0]);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk; kt0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int kt = kt0 + d;
      if (kt >= nk) break;
      compute(kt & 1);
      // slab kt+1 (in ring slot d+1) goes to the other LDS buffer, whose
      // readers passed the previous barrier; ring slot d, whose slab is
      // already in LDS, is refilled with slab kt+DEPTH
      store_slab((kt + 1) & 1, ra[(d + 1) % DEPTH], rb[(d + 1) % DEPTH]);
      load_slab(min(kt + DEPTH, nk - 1) * kBK, ra[d], rb[d]);
      __syncthreads();
    }
  }

  // Epilogue: register e of lane (j, hh) is row 8(e/4) + 4hh + e%4 of the
  // 32x32 block, column j; columns past Nout are the U = x A^T columns.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int m0 = m_blk + wm + 32 * i, n0 = n_blk + wn + 32 * j;
      const int col = n0 + lane32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (row >= p.M) continue;
        if (col < p.Nout)
          p.y[static_cast<long>(row) * p.Nout + col] = acc[i][j][e];
        else if (col < p.Nout + p.r)
          p.u[static_cast<long>(row) * p.r + (col - p.Nout)] = acc[i][j][e];
      }
    }
}

// y[m] += scale * (U B^T)[m] on MASK rows only, one wave per 32x32 tile of
// y; tiles without a MASK row are skipped. U (fp32) is split into bf16 high
// and low halves, so the product runs on bf16 MFMA (32x32x16) with both
// operands read as 16-byte runs. Every load of a wave (its mask bytes, all of
// U and B for the tile, then y of its MASK rows) is issued before the first
// MFMA, so a tile costs about two memory round trips. Clean rows are never
// written.
struct DeltaParams {
  const float* u;      // [M][r]
  const uint16_t* b;   // [Nout][r]
  const uint8_t* mask; // [M]
  float* y;            // [M][Nout]
  int M, Nout, r;
  float scale;
};

template <int R16>  // r / 16
__global__ __launch_bounds__(256) void lora_delta_kernel(DeltaParams p) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lane32 = lane & 31, hh = lane >> 5;
  const int tiles_n = (p.Nout + 31) / 32;
  const long tile = static_cast<long>(blockIdx.x) * 4 + wave;
  if (tile >= static_cast<long>((p.M + 31) / 32) * tiles_n) return;
  const int m0 = static_cast<int>(tile / tiles_n) * 32, n0 = static_cast<int>(tile % tiles_n) * 32;
  const int arow = m0 + lane32, bcol = n0 + lane32;
  const int mine = arow < p.M ? p.mask[arow] != 0 : 0;
  if (!__any(mine)) return;

  f32x4 uv[R16][2];
  u32x4 bv[R16];
#pragma unroll
  for (int k = 0; k < R16; ++k) {
    if (arow < p.M) {
      const f32x4* src = reinterpret_cast<const f32x4*>(p.u + static_cast<long>(arow) * p.r + 16 * k + 8 * hh);
      uv[k][0] = src[0];
      uv[k][1] = src[1];
    } else {
      uv[k][0] = uv[k][1] = f32x4{};
    }
    bv[k] = bcol < p.Nout ? *reinterpret_cast<const u32x4*>(p.b + static_cast<long>(bcol) * p.r + 16 * k + 8 * hh)
                          : u32x4{0, 0, 0, 0};
  }
  // register e holds row 8(e/4) + 4hh + e%4 of the tile; its mask bit sits
  // in the lane whose U row that is
  float yv[16];
  int live = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rl = 8 * (e >> 2) + 4 * hh + (e & 3);
    const int on = __shfl(mine, rl) && bcol < p.Nout;
    live |= on << e;
    yv[e] = on ? p.y[static_cast<long>(m0 + rl) * p.Nout + bcol] : 0.f;
  }

  f32x16 dl = {};
#pragma unroll
  for (int k = 0; k < R16; ++k) {
    const float f[8] = {uv[k][0][0], uv[k][0][1], uv[k][0][2], uv[k][0][3],
                        uv[k][1][0], uv[k][1][1], uv[k][1][2], uv[k][1][3]};
    u32x4 hi, lo;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t ua = __float_as_uint(f[2 * t]) & 0xffff0000u, ub = __float_as_uint(f[2 * t + 1]) & 0xffff0000u;
      hi[t] = (ua >> 16) | ub;
      lo[t] = f32_to_bf16_bits(f[2 * t] - __uint_as_float(ua)) |
              (f32_to_bf16_bits(f[2 * t + 1] - __uint_as_float(ub)) << 16);
    }
    const bf16x8 bb = __builtin_bit_cast(bf16x8, bv[k]);
    dl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi), bb, dl, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo), bb, dl, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if ((live >> e) & 1) {
      const int rl = 8 * (e >> 2) + 4 * hh + (e & 3);
      p.y[static_cast<long>(m0 + rl) * p.Nout + bcol] = fmaf(p.scale, dl[e], yv[e]);
    }
  }
}

}  // namespace isd

// ================================================================ host API
namespace {
using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Tile choice depends only on (M, output columns) and the CU count, never on
// the data, and every choice gives each output the same reduction order.
// 128x128 when that still gives one workgroup per CU. Otherwise 64x64 when
// its workgroups spread evenly over the CUs (or fit in one round), else
// 128x64: a CU that holds one 64x64 workgroup more than the others sets the
// pace, because four resident 64x64 workgroups saturate its LDS bandwidth.
constexpr int kDepth = 3;  // K slabs in flight per thread

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  const int cols = p.Nout + (p.a ? p.r : 0);
  const long cus = isd_device_cus_internal();
  const long big = static_cast<long>((p.M + 127) / 128) * ((cols + 127) / 128);
  const long small = static_cast<long>((p.M + 63) / 64) * ((cols + 63) / 64);
  auto tiles = [&](int bm, int bn) { return dim3(static_cast<unsigned>(((p.M + bm - 1) / bm) * ((cols + bn - 1) / bn))); };
  if (big >= cus) {
    hipLaunchKernelGGL((gemm_nt_kernel<64, 64, kDepth>), tiles(128, 128), dim3(256), 0, stream, p);
  } else if (small <= cus || small % cus == 0) {
    hipLaunchKernelGGL((gemm_nt_kernel<32, 32, kDepth>), tiles(64, 64), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<64, 32, kDepth>), tiles(128, 64), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_delta(const float* U, const void* B, const uint8_t* mask, int M, int Nout, int r, float scale,
                        float* y, hipStream_t stream) {
  DeltaParams d{};
  d.u = U;
  d.b = static_cast<const uint16_t*>(B);
  d.mask = mask;
  d.y = y;
  d.M = M;
  d.Nout = Nout;
  d.r = r;
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

int check_gemm_args(const void* x, const void* W, int M, int K, int Nout, const float* y) {
  if (M < 0 || K < 0 || Nout < 0) return ISD_E_INVALID;
  if (M == 0 || Nout == 0) return ISD_OK;
  if (!x || !W || !y) return ISD_E_INVALID;
  if (K == 0 || K % kBK != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W)) return ISD_E_INVALID;
  return ISD_OK;
}

int check_lora_args(const void* A, const void* B, const uint8_t* mask, int r, void* ws, size_t ws_bytes, int M) {
  if (!A || !B || !mask) return ISD_E_INVALID;
  if (r < 16 || r > 128 || r % 16 != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(A) || !aligned16(B)) return ISD_E_INVALID;
  const size_t need = static_cast<size_t>(M) * r * sizeof(float);
  if (!ws || ws_bytes < need || !aligned16(ws)) return ISD_E_WORKSPACE;
  return ISD_OK;
}

}  // namespace

extern "C" {

int isd_linear(const void* x, const void* W, int M, int K, int Nout, float* y, hipStream_t stream) {
  int rc = check_gemm_args(x, W, M, K, Nout, y);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(W);
  p.y = y;
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  return launch_gemm(p, stream) == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

size_t isd_lora_workspace_size(int M, int r) {
  if (M < 0 || r < 0) return 0;
  return static_cast<size_t>(M) * r * sizeof(float);
}

int gated_lora_apply(const void* x, const void* A, const void* B, const uint8_t* is_mask, int M, int K, int Nout,
                     int r, float scale, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_args(x, A, M, K, Nout, y);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  // U = x A^T through the projection GEMM (A's rows as the output columns),
  // so U is bit-identical to the U columns of the fused call below.
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(A);
  p.y = static_cast<float*>(ws);
  p.M = M;
  p.K = K;
  p.Nout = r;
  if (launch_gemm(p, stream) != hipSuccess) return ISD_E_LAUNCH;
  return launch_delta(static_cast<const float*>(ws), B, is_mask, M, Nout, r, scale, y, stream) == hipSuccess
             ? ISD_OK
             : ISD_E_LAUNCH;
}

int isd_linear_gated(const void* x, const void* W, const void* A, const void* B, const uint8_t* is_mask, int M, int K,
                     int Nout, int r, float scale, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_args(x, W, M, K, Nout, y);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(W);
  p.a = static_cast<const uint16_t*>(A);
  p.y = y;
  p.u = static_cast<float*>(ws);
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  p.r = r;
  if (launch_gemm(p, stream) != hipSuccess) return ISD_E_LAUNCH;
  return launch_delta(static_cast<const float*>(ws), B, is_mask, M, Nout, r, scale, y, stream) == hipSuccess
             ? ISD_OK
             : ISD_E_LAUNCH;
}

}  // extern "C"

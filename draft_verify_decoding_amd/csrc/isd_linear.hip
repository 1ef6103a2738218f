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
// in 32x32 MFMA blocks), K in steps of 64 through double-buffered LDS with
// padded rows (72 elements) so the 16-byte operand reads are conflict-free.
// The per-output reduction order is K-step by K-step in ascending K and does
// not depend on M, the tile choice, the other rows or the mask.
// LoRA: U = x A^T (same GEMM, fp32 out), then delta = U B^T on MFMA
// 32x32x2 f32 (B widened exactly), added with one fma only to MASK rows.
#include "isd_common.hpp"

namespace isd {

constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // elements per LDS row

// delta tile (rows m0.., cols n0..) = U[m0:m0+32][0:r] . B[n0:n0+32][0:r]^T in
// the 32x32 MFMA accumulator layout: register e of lane (j, hh) is row
// m0 + 8(e/4) + 4hh + e%4, column n0 + j.
__device__ __forceinline__ f32x16 lora_delta_tile(const float* U, int r, const uint16_t* B, int m0, int n0, int M,
                                                  int Nout, int lane) {
  const int i = lane & 31, hh = lane >> 5;
  const int row = m0 + i, col = n0 + i;
  f32x16 acc = {};
  for (int s = 0; s < r / 2; ++s) {
    const int k = 2 * s + hh;
    const float a = row < M ? U[static_cast<long>(row) * r + k] : 0.f;
    const float bb = col < Nout ? bf16_bits_to_f32(B[static_cast<long>(col) * r + k]) : 0.f;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bb, acc, 0, 0, 0);
  }
  return acc;
}

struct GemmParams {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [Nout][K]
  float* y;           // [M][Nout]
  int M, K, Nout;
  // gated epilogue
  const float* U;        // [M][r]
  const uint16_t* B;     // [Nout][r]
  const uint8_t* mask;   // [M]
  int r;
  float scale;
};

template <int WM, int WN, bool GATED>
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
  const int m_blk = blockIdx.y * BM, n_blk = blockIdx.x * BN;

  // Global->register staging: thread loads rows (tid / 8) + 32*q, 16 bytes at
  // column 8 * (tid % 8) of the 64-wide K slab.
  const int ld_row = tid >> 3, ld_col = (tid & 7) * 8;
  u32x4 ra[A_ROUNDS], rb[B_ROUNDS];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int q = 0; q < A_ROUNDS; ++q) {
      const int row = m_blk + ld_row + 32 * q;
      ra[q] = row < p.M ? *reinterpret_cast<const u32x4*>(p.x + static_cast<long>(row) * p.K + k0 + ld_col)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < B_ROUNDS; ++q) {
      const int row = n_blk + ld_row + 32 * q;
      rb[q] = row < p.Nout ? *reinterpret_cast<const u32x4*>(p.w + static_cast<long>(row) * p.K + k0 + ld_col)
                           : u32x4{0, 0, 0, 0};
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int q = 0; q < A_ROUNDS; ++q)
      *reinterpret_cast<u32x4*>(&sA[buf][(ld_row + 32 * q) * kLdsStride + ld_col]) = ra[q];
#pragma unroll
    for (int q = 0; q < B_ROUNDS; ++q)
      *reinterpret_cast<u32x4*>(&sB[buf][(ld_row + 32 * q) * kLdsStride + ld_col]) = rb[q];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = p.K / kBK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab((kt + 1) * kBK);
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
    if (kt + 1 < nk) {
      store_slab(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: register e of lane (j, hh) is row 8(e/4) + 4hh + e%4 of the
  // 32x32 block, column j.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int m0 = m_blk + wm + 32 * i, n0 = n_blk + wn + 32 * j;
      if constexpr (GATED) {
        bool any = false;
        const int rrow = m0 + lane32;
        if (rrow < p.M) any = p.mask[rrow] != 0;
        if (__any(any)) {
          const f32x16 dl = lora_delta_tile(p.U, p.r, p.B, m0, n0, p.M, p.Nout, lane);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (row < p.M && p.mask[row]) acc[i][j][e] = fmaf(p.scale, dl[e], acc[i][j][e]);
          }
        }
      }
      const int col = n0 + lane32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (row < p.M && col < p.Nout) p.y[static_cast<long>(row) * p.Nout + col] = acc[i][j][e];
      }
    }
}

// y[m] += scale * delta on MASK rows only, one wave per 32x32 tile.
__global__ __launch_bounds__(256) void lora_delta_kernel(GemmParams p) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, hh = lane >> 5;
  const int tiles_n = (p.Nout + 31) / 32;
  const long tile = static_cast<long>(blockIdx.x) * 4 + wave;
  if (tile >= static_cast<long>((p.M + 31) / 32) * tiles_n) return;
  const int m0 = static_cast<int>(tile / tiles_n) * 32, n0 = static_cast<int>(tile % tiles_n) * 32;
  const int rrow = m0 + (lane & 31);
  const bool mine = rrow < p.M && p.mask[rrow] != 0;
  if (!__any(mine)) return;
  const f32x16 dl = lora_delta_tile(p.U, p.r, p.B, m0, n0, p.M, p.Nout, lane);
  const int col = n0 + (lane & 31);
  if (col >= p.Nout) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = m0 + 8 * (e >> 2) + 4 * hh + (e & 3);
    if (row < p.M && p.mask[row]) {
      float* yp = p.y + static_cast<long>(row) * p.Nout + col;
      *yp = fmaf(p.scale, dl[e], *yp);
    }
  }
}

// U = x A^T for the LoRA (r <= 128 columns): split-K over kUSplit slices so
// a 512 x 4096 problem still spreads over 128 workgroups. Each wave reduces
// a quarter of its slice, the waves are summed in order through LDS, and the
// slices are summed in order by lora_u_reduce_kernel: a fixed reduction
// order for every element whatever M is.
constexpr int kUSplit = 8;

__global__ __launch_bounds__(256) void lora_u_partial_kernel(const uint16_t* x, const uint16_t* A, float* upart,
                                                             int M, int K, int r) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lane32 = lane & 31, hh = lane >> 5;
  const int m0 = blockIdx.x * 32, ks = blockIdx.y;
  // k-steps of 16 split evenly over the kUSplit * 4 waves of the grid row
  const int T = K / 16, gw = ks * 4 + wave;
  const int s_begin = (gw * T) / (kUSplit * 4), s_end = ((gw + 1) * T) / (kUSplit * 4);
  const int row = m0 + lane32;
  const int nblk = (r + 31) / 32;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int st = s_begin; st < s_end; ++st) {
    const int k = 16 * st;
    const u32x4 av = row < M ? *reinterpret_cast<const u32x4*>(x + static_cast<long>(row) * K + k + 8 * hh)
                             : u32x4{0, 0, 0, 0};
    const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nblk) {
        const int col = 32 * j + lane32;
        const u32x4 bv = col < r ? *reinterpret_cast<const u32x4*>(A + static_cast<long>(col) * K + k + 8 * hh)
                                 : u32x4{0, 0, 0, 0};
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
      }
    }
  }
  __shared__ float red[4][32][129];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < nblk)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave][8 * (e >> 2) + 4 * hh + (e & 3)][32 * j + lane32] = acc[j][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * r; idx += 256) {
    const int i = idx / r, c = idx % r;
    if (m0 + i >= M) continue;
    const float v = ((red[0][i][c] + red[1][i][c]) + red[2][i][c]) + red[3][i][c];
    upart[(static_cast<long>(ks) * M + m0 + i) * r + c] = v;
  }
}

__global__ __launch_bounds__(256) void lora_u_reduce_kernel(const float* upart, float* U, int M, int r) {
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(M) * r) return;
  float v = upart[idx];
#pragma unroll
  for (int ks = 1; ks < kUSplit; ++ks) v += upart[static_cast<long>(ks) * M * r + idx];
  U[idx] = v;
}

}  // namespace isd

// ================================================================ host API
namespace {
using namespace isd;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Tile choice depends only on the problem's (M, Nout): the largest of
// 128x128, 128x64 and 64x64 that still gives one workgroup per CU. The
// reduction order inside a tile is the same for every choice.
template <bool GATED>
hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  auto wgs = [&](int bm, int bn) { return static_cast<long>((p.M + bm - 1) / bm) * ((p.Nout + bn - 1) / bn); };
  if (wgs(128, 128) >= 256) {
    hipLaunchKernelGGL((gemm_nt_kernel<64, 64, GATED>), dim3((p.Nout + 127) / 128, (p.M + 127) / 128), dim3(256),
                       0, stream, p);
  } else if (wgs(128, 64) >= 256) {
    hipLaunchKernelGGL((gemm_nt_kernel<64, 32, GATED>), dim3((p.Nout + 63) / 64, (p.M + 127) / 128), dim3(256), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<32, 32, GATED>), dim3((p.Nout + 63) / 64, (p.M + 63) / 64), dim3(256), 0,
                       stream, p);
  }
  return hipGetLastError();
}

// U = x A^T into ws (the first M*r floats), split-K partials after it.
hipError_t launch_lora_u(const void* x, const void* A, int M, int K, int r, void* ws, hipStream_t stream) {
  float* U = static_cast<float*>(ws);
  float* upart = U + static_cast<size_t>(M) * r;
  hipLaunchKernelGGL(lora_u_partial_kernel, dim3((M + 31) / 32, kUSplit), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(A), upart, M, K, r);
  const long n = static_cast<long>(M) * r;
  hipLaunchKernelGGL(lora_u_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, upart,
                     U, M, r);
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
  if (!aligned16(A)) return ISD_E_INVALID;
  const size_t need = static_cast<size_t>(M) * r * sizeof(float) * (1 + kUSplit);
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
  return launch_gemm<false>(p, stream) == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

size_t isd_lora_workspace_size(int M, int r) {
  if (M < 0 || r < 0) return 0;
  return static_cast<size_t>(M) * r * sizeof(float) * (1 + kUSplit);
}

int gated_lora_apply(const void* x, const void* A, const void* B, const uint8_t* is_mask, int M, int K, int Nout,
                     int r, float scale, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_args(x, A, M, K, Nout, y);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  if (launch_lora_u(x, A, M, K, r, ws, stream) != hipSuccess) return ISD_E_LAUNCH;
  GemmParams p{};
  p.y = y;
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  p.U = static_cast<const float*>(ws);
  p.B = static_cast<const uint16_t*>(B);
  p.mask = is_mask;
  p.r = r;
  p.scale = scale;
  const long tiles = static_cast<long>((M + 31) / 32) * ((Nout + 31) / 32);
  hipLaunchKernelGGL(lora_delta_kernel, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

int isd_linear_gated(const void* x, const void* W, const void* A, const void* B, const uint8_t* is_mask, int M, int K,
                     int Nout, int r, float scale, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_args(x, W, M, K, Nout, y);
  if (rc || M == 0 || Nout == 0) return rc;
  rc = check_lora_args(A, B, is_mask, r, ws, ws_bytes, M);
  if (rc) return rc;
  rc = isd_check_device_internal();
  if (rc) return rc;
  if (launch_lora_u(x, A, M, K, r, ws, stream) != hipSuccess) return ISD_E_LAUNCH;
  GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(W);
  p.y = y;
  p.M = M;
  p.K = K;
  p.Nout = Nout;
  p.U = static_cast<const float*>(ws);
  p.B = static_cast<const uint16_t*>(B);
  p.mask = is_mask;
  p.r = r;
  p.scale = scale;
  return launch_gemm<true>(p, stream) == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // extern "C"

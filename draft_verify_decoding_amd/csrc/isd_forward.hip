// The elementwise and normalisation steps of the forward around the ISD
// step (gfx950): RMSNorm with the residual add folded in, bf16 casts that
// split a fused projection output, and the SwiGLU activation.
//
// The pages name the base models of I-DLM (Qwen3-8B / 32B, I-DLM page on
// fr.news.hada.io, "Documentation et ressources > Model Zoo") and say that
// one causal forward verifies and proposes ("Methodologie d'I-DLM"); they do
// not describe the decoder block. These are the pieces of the usual
// pre-norm block of that family that the projections, the attention and the
// LM head of this library do not already cover. All of them stream HBM once
// (one read of every input, one write of every output), in 16-byte accesses.
#include "isd_common.hpp"

namespace isd {

constexpr int kNormThreads = 256;

// fp32 -> bf16 (round to nearest even) of 4 values, packed in two words.
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16), f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16));
}

// One workgroup per row: h[m] += delta[m] (when given), then
// out[m] = bf16(h[m] / sqrt(mean(h[m]^2) + eps) * gamma). The mean square is
// a fixed-order reduction (per thread, then a wave butterfly, then the four
// waves in order), so a row's result does not depend on the other rows.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float* h, const float* delta, const uint16_t* gamma,
                                                               int H, float eps, uint16_t* out) {
  __shared__ float s_part[kNormThreads / kWave];
  const int m = blockIdx.x;
  float* row = h + static_cast<long>(m) * H;
  const float* drow = delta ? delta + static_cast<long>(m) * H : nullptr;
  // H is a multiple of 4 * 256 = 1024 or handled by the tail loop below
  float ss = 0.f;
  for (int c = 4 * threadIdx.x; c < H; c += 4 * kNormThreads) {
    f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    if (drow) {
      const f32x4 d = *reinterpret_cast<const f32x4*>(drow + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = v[k] + d[k];
      *reinterpret_cast<f32x4*>(row + c) = v;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = fmaf(v[k], v[k], ss);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) ss += __shfl_xor(ss, off, kWave);
  if (threadIdx.x % kWave == 0) s_part[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = s_part[0];
#pragma unroll
  for (int i = 1; i < kNormThreads / kWave; ++i) tot += s_part[i];
  const float inv = 1.f / sqrtf(tot / static_cast<float>(H) + eps);
  for (int c = 4 * threadIdx.x; c < H; c += 4 * kNormThreads) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);  // this thread's own (updated) values
    const uint2 g = *reinterpret_cast<const uint2*>(gamma + c);
    const float g0 = bf16_lo(g.x), g1 = bf16_hi(g.x), g2 = bf16_lo(g.y), g3 = bf16_hi(g.y);
    *reinterpret_cast<uint2*>(out + static_cast<long>(m) * H + c) =
        pack4_bf16(v[0] * inv * g0, v[1] * inv * g1, v[2] * inv * g2, v[3] * inv * g3);
  }
}

// Column-split cast: columns [c0_p, c0_p + w_p) of src [M][ld] (fp32) go,
// rounded to bf16, to dst_p [M][w_p] (contiguous), for up to four parts.
struct CastParts {
  uint16_t* dst[4];
  int c0[4], w[4];
  int n;
};

__global__ __launch_bounds__(256) void cast_split_kernel(const float* src, long ld, int M, int ncols, CastParts parts) {
  const long i = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) * 4;  // first of 4 columns
  if (i >= static_cast<long>(M) * ncols) return;
  const int m = static_cast<int>(i / ncols), c = static_cast<int>(i % ncols);
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + static_cast<long>(m) * ld + c);
  int pi = 0;
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (k < parts.n && c >= parts.c0[k]) pi = k;
  const int cc = c - parts.c0[pi];
  *reinterpret_cast<uint2*>(parts.dst[pi] + static_cast<long>(m) * parts.w[pi] + cc) = pack4_bf16(v[0], v[1], v[2], v[3]);
}

// out[m][i] = bf16(silu(gu[m][i]) * gu[m][I + i]) with silu(z) = z / (1 + e^-z).
__global__ __launch_bounds__(256) void swiglu_kernel(const float* gu, int M, int I, uint16_t* out) {
  const long i = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= static_cast<long>(M) * I) return;
  const int m = static_cast<int>(i / I), c = static_cast<int>(i % I);
  const float* row = gu + static_cast<long>(m) * 2 * I;
  const f32x4 g = *reinterpret_cast<const f32x4*>(row + c);
  const f32x4 u = *reinterpret_cast<const f32x4*>(row + I + c);
  float a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = g[k] / (1.f + fast_exp2(-g[k] * kLog2e)) * u[k];
  *reinterpret_cast<uint2*>(out + static_cast<long>(m) * I + c) = pack4_bf16(a[0], a[1], a[2], a[3]);
}

}  // namespace isd

namespace {
bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool aligned8(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 7u) == 0; }
}  // namespace

extern "C" {

int isd_rmsnorm(float* h, const float* delta, const void* gamma, int M, int H, float eps, void* out,
                hipStream_t stream) {
  if (M < 0 || H < 0 || !(eps >= 0.f)) return ISD_E_INVALID;
  if (M == 0) return ISD_OK;
  if (!h || !gamma || !out) return ISD_E_INVALID;
  if (H == 0 || H % 4 != 0) return ISD_E_UNSUPPORTED;
  if (!aligned16(h) || (delta && !aligned16(delta)) || !aligned8(gamma) || !aligned8(out)) return ISD_E_INVALID;
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  hipLaunchKernelGGL(isd::rmsnorm_kernel, dim3(M), dim3(isd::kNormThreads), 0, stream, h, delta,
                     static_cast<const uint16_t*>(gamma), H, eps, static_cast<uint16_t*>(out));
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

int isd_cast_bf16(const float* src, int64_t ld, int M, int nparts, const int* widths, void* const* dst,
                  hipStream_t stream) {
  if (M < 0 || nparts < 1 || nparts > 4 || !widths || !dst) return ISD_E_INVALID;
  isd::CastParts parts{};
  int ncols = 0;
  for (int k = 0; k < nparts; ++k) {
    if (widths[k] <= 0 || widths[k] % 4 != 0 || !dst[k] || !aligned8(dst[k])) return ISD_E_INVALID;
    parts.dst[k] = static_cast<uint16_t*>(dst[k]);
    parts.c0[k] = ncols;
    parts.w[k] = widths[k];
    ncols += widths[k];
  }
  parts.n = nparts;
  if (M == 0) return ISD_OK;
  if (!src || ld < ncols || ld % 4 != 0 || !aligned16(src)) return ISD_E_INVALID;
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  const long n4 = static_cast<long>(M) * ncols / 4;
  hipLaunchKernelGGL(isd::cast_split_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, stream, src,
                     static_cast<long>(ld), M, ncols, parts);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

int isd_swiglu(const float* gu, int M, int I, void* out, hipStream_t stream) {
  if (M < 0 || I < 0) return ISD_E_INVALID;
  if (M == 0 || I == 0) return ISD_OK;
  if (!gu || !out || I % 4 != 0 || !aligned16(gu) || !aligned8(out)) return ISD_E_INVALID;
  const int rc = isd_check_device_internal();
  if (rc) return rc;
  const long n4 = static_cast<long>(M) * I / 4;
  hipLaunchKernelGGL(isd::swiglu_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, stream, gu, M, I,
                     static_cast<uint16_t*>(out));
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_E_LAUNCH;
}

}  // extern "C"

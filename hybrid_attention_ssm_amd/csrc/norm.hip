// Fusion of the two branches (Hymba paper §2.1 Eq. (3) with the "average"
// of its text and the mean fusion of Appendix B):
//   F = 1/2 [beta_attn * O / rms(O) || beta_ssm * Y / rms(Y)],
//   rms(v) = sqrt(mean(v^2) + eps), statistics in fp32.
// One wavefront (or, for few rows, one workgroup) per token row; the two
// halves are written side by side so a
// single output projection over [H*hd + D] columns follows.
#include "hh_internal.h"

namespace hh {

namespace {
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <class T> struct Vec;
template <> struct Vec<bf16> { static constexpr int W = 8; typedef bf16x8 type; };
template <> struct Vec<float> { static constexpr int W = 4; typedef f32x4 type; };

// partial sums over this lane's elements; lanes of WPR waves stride the row
template <class T, int WPR>
__device__ __forceinline__ float sumsq(const T *p, int n, int lane) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  float s = 0.0f;
  for (int i = lane * W; i < n; i += 64 * WPR * W) {
    const V v = *reinterpret_cast<const V *>(p + i);
#pragma unroll
    for (int e = 0; e < W; ++e) { const float f = to_f32(v[e]); s = fmaf(f, f, s); }
  }
  return wave_sum(s);
}

template <class T, int WPR>
__device__ __forceinline__ void scaled(const T *p, const float *beta, float r, T *dst, int n, int lane) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  for (int i = lane * W; i < n; i += 64 * WPR * W) {
    const V v = *reinterpret_cast<const V *>(p + i);
    V o;
#pragma unroll
    for (int e = 0; e < W; ++e) o[e] = from_f32<T>(0.5f * beta[i + e] * to_f32(v[e]) * r);
    *reinterpret_cast<V *>(dst + i) = o;
  }
}
}  // namespace

// WPR waves per token row (1 for long inputs, 4 when there are few rows);
// 256 threads per workgroup
template <class T, int WPR>
__global__ void __launch_bounds__(256) norm_fuse(NormArgs a) {
  __shared__ float part[4][2];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (4 / WPR) + wave / WPR;
  const int lane = (wave % WPR) * 64 + (threadIdx.x & 63);
  const bool live = row < a.rows;
  const int r = live ? row : 0;
  const T *o = reinterpret_cast<const T *>(a.o) + (size_t)r * a.Wa;
  const T *y = reinterpret_cast<const T *>(a.y) + (size_t)r * a.D;
  T *f = reinterpret_cast<T *>(a.f) + (size_t)r * (a.Wa + a.D);
  float so = sumsq<T, WPR>(o, a.Wa, lane);
  float sy = sumsq<T, WPR>(y, a.D, lane);
  if (WPR > 1) {
    if ((threadIdx.x & 63) == 0) { part[wave][0] = so; part[wave][1] = sy; }
    __syncthreads();
    so = 0.0f; sy = 0.0f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) { so += part[w][0]; sy += part[w][1]; }
  }
  if (!live) return;
  const float ro = 1.0f / sqrtf(so / (float)a.Wa + a.eps);
  const float ry = 1.0f / sqrtf(sy / (float)a.D + a.eps);
  scaled<T, WPR>(o, a.beta_attn, ro, f, a.Wa, lane);
  scaled<T, WPR>(y, a.beta_ssm, ry, f + a.Wa, a.D, lane);
}

// Same computation with each lane's chunks of the row held in registers: all
// loads of a row are issued before the first use, and the row is read once.
// Lanes of WPR waves take chunks lane, lane + 64*WPR, ... (MAXC at most).
template <class T, int WPR, int MAXC>
__global__ void __launch_bounds__(256) norm_fuse_reg(NormArgs a) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  __shared__ float part[4][2];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (4 / WPR) + wave / WPR;
  const int lane = (wave % WPR) * 64 + (threadIdx.x & 63);
  const bool live = row < a.rows;
  const int r = live ? row : 0;
  const T *o = reinterpret_cast<const T *>(a.o) + (size_t)r * a.Wa;
  const T *y = reinterpret_cast<const T *>(a.y) + (size_t)r * a.D;
  T *f = reinterpret_cast<T *>(a.f) + (size_t)r * (a.Wa + a.D);
  const int no = a.Wa / W, ny = a.D / W;
  V vo[MAXC], vy[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {   // indices past the row repeat its last chunk
    vo[j] = *reinterpret_cast<const V *>(o + (size_t)min(lane + j * 64 * WPR, no - 1) * W);
    vy[j] = *reinterpret_cast<const V *>(y + (size_t)min(lane + j * 64 * WPR, ny - 1) * W);
  }
  float so = 0.0f, sy = 0.0f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    float po = 0.0f, py = 0.0f;
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const float fo = to_f32(vo[j][e]), fy = to_f32(vy[j][e]);
      po = fmaf(fo, fo, po);
      py = fmaf(fy, fy, py);
    }
    if (lane + j * 64 * WPR < no) so += po;
    if (lane + j * 64 * WPR < ny) sy += py;
  }
  so = wave_sum(so);
  sy = wave_sum(sy);
  if (WPR > 1) {
    if ((threadIdx.x & 63) == 0) { part[wave][0] = so; part[wave][1] = sy; }
    __syncthreads();
    so = 0.0f; sy = 0.0f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) { so += part[w][0]; sy += part[w][1]; }
  }
  if (!live) return;
  const float ro = 0.5f / sqrtf(so / (float)a.Wa + a.eps);
  const float ry = 0.5f / sqrtf(sy / (float)a.D + a.eps);
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int io = lane + j * 64 * WPR;
    if (io < no) {
      V out;
#pragma unroll
      for (int e = 0; e < W; ++e) out[e] = from_f32<T>(a.beta_attn[io * W + e] * to_f32(vo[j][e]) * ro);
      *reinterpret_cast<V *>(f + (size_t)io * W) = out;
    }
    const int iy = lane + j * 64 * WPR;
    if (iy < ny) {
      V out;
#pragma unroll
      for (int e = 0; e < W; ++e) out[e] = from_f32<T>(a.beta_ssm[iy * W + e] * to_f32(vy[j][e]) * ry);
      *reinterpret_cast<V *>(f + a.Wa + (size_t)iy * W) = out;
    }
  }
}

template <class T>
hipError_t launch_norm_fuse(const NormArgs &a, hipStream_t s) {
  constexpr int W = Vec<T>::W;
  constexpr int MAXC = 8;
  const int widest = std::max(a.Wa, a.D) / W;
  if (a.Wa % W == 0 && a.D % W == 0) {
    if (a.rows < 2048 && widest <= MAXC * 256) {
      hipLaunchKernelGGL((norm_fuse_reg<T, 4, MAXC>), dim3(a.rows), dim3(256), 0, s, a);
      return hipGetLastError();
    }
    if (widest <= MAXC * 64) {
      hipLaunchKernelGGL((norm_fuse_reg<T, 1, MAXC>), dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.rows < 2048)
    hipLaunchKernelGGL((norm_fuse<T, 4>), dim3(a.rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((norm_fuse<T, 1>), dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_norm_fuse<float>(const NormArgs &, hipStream_t);
template hipError_t launch_norm_fuse<bf16>(const NormArgs &, hipStream_t);

}  // namespace hh

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

// block 0 records the length of a producer's cache (see NormArgs): the
// prompt's length after a prefill, one more token after a decode step
__device__ __forceinline__ void record_len(const NormArgs &a) {
  if (blockIdx.x != 0) return;
  if (a.set_len)
    for (int i = threadIdx.x; i < a.set_len_n; i += blockDim.x) a.set_len[i] = a.set_len_value;
  if (a.len_bump)
    for (int i = threadIdx.x; i < a.bump_n; i += blockDim.x)
      if (a.bump_ring || a.len_bump[i] < a.bump_cap) a.len_bump[i] += 1;
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
  record_len(a);
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
  record_len(a);
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

// Decode: the attention half arrives as the split partials of the decode
// attention (per head and split: m, l, a[hd], see launch_decode_attention).
// Scaling split s by 2^(m_s - max m) and summing gives O = sum a / sum l, the
// same softmax-weighted mean of V over all keys; O is rounded to T exactly as
// a stored O would be, then normalised like above.  One workgroup per row;
// thread t merges the W-wide column groups t, t + 256, ... (C at most).
template <class T, int C>
__global__ void __launch_bounds__(256) norm_fuse_parts(NormArgs a) {
  record_len(a);
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  __shared__ float part[4][2];
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const int no = a.Wa / W, ny = a.D / W, per_head = a.hd / W, stride = a.hd + 2;
  const float *pr = a.part + (size_t)row * a.H * a.nsplit * stride;
  const T *y = reinterpret_cast<const T *>(a.y) + (size_t)row * a.D;
  T *f = reinterpret_cast<T *>(a.f) + (size_t)row * (a.Wa + a.D);
  V vy[C];
#pragma unroll
  for (int j = 0; j < C; ++j)   // indices past the row repeat its last chunk
    vy[j] = *reinterpret_cast<const V *>(y + (size_t)min(tid + j * 256, ny - 1) * W);
  float vo[C][W];
  float so = 0.0f, sy = 0.0f;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int u = tid + j * 256;
#pragma unroll
    for (int e = 0; e < W; ++e) vo[j][e] = 0.0f;
    if (u < no) {
      const float *ph = pr + (size_t)(u / per_head) * a.nsplit * stride;
      const int c = (u % per_head) * W;
      float M = -INFINITY, L = 0.0f, acc[W];
#pragma unroll
      for (int e = 0; e < W; ++e) acc[e] = 0.0f;
#pragma unroll 4
      for (int sp = 0; sp < a.nsplit; ++sp) {
        const float *q = ph + (size_t)sp * stride;
        const float ms = q[0], ls = q[1];
        float av[W];
#pragma unroll
        for (int e = 0; e < W; e += 2) {   // a[] is 8-byte aligned
          const float2 t = *reinterpret_cast<const float2 *>(q + 2 + c + e);
          av[e] = t.x; av[e + 1] = t.y;
        }
        const float mn = fmaxf(M, ms);
        const float sc_old = M == -INFINITY ? 0.0f : exp2_fast(M - mn);
        const float sc_new = ms == -INFINITY ? 0.0f : exp2_fast(ms - mn);
        L = L * sc_old + ls * sc_new;
#pragma unroll
        for (int e = 0; e < W; ++e) acc[e] = acc[e] * sc_old + av[e] * sc_new;
        M = mn;
      }
      const float inv = 1.0f / L;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        vo[j][e] = to_f32(from_f32<T>(acc[e] * inv));
        so = fmaf(vo[j][e], vo[j][e], so);
      }
    }
    if (u < ny) {
#pragma unroll
      for (int e = 0; e < W; ++e) { const float fy = to_f32(vy[j][e]); sy = fmaf(fy, fy, sy); }
    }
  }
  so = wave_sum(so);
  sy = wave_sum(sy);
  if ((tid & 63) == 0) { part[wave][0] = so; part[wave][1] = sy; }
  __syncthreads();
  so = part[0][0] + part[1][0] + part[2][0] + part[3][0];
  sy = part[0][1] + part[1][1] + part[2][1] + part[3][1];
  const float ro = 0.5f / sqrtf(so / (float)a.Wa + a.eps);
  const float ry = 0.5f / sqrtf(sy / (float)a.D + a.eps);
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int u = tid + j * 256;
    if (u < no) {
      V out;
#pragma unroll
      for (int e = 0; e < W; ++e) out[e] = from_f32<T>(a.beta_attn[u * W + e] * vo[j][e] * ro);
      *reinterpret_cast<V *>(f + (size_t)u * W) = out;
    }
    if (u < ny) {
      V out;
#pragma unroll
      for (int e = 0; e < W; ++e) out[e] = from_f32<T>(a.beta_ssm[u * W + e] * to_f32(vy[j][e]) * ry);
      *reinterpret_cast<V *>(f + a.Wa + (size_t)u * W) = out;
    }
  }
}

template <class T>
hipError_t launch_norm_fuse(const NormArgs &a, hipStream_t s) {
  constexpr int W = Vec<T>::W;
  constexpr int MAXC = 8;
  if (a.part) {
    if (a.Wa % W || a.D % W || a.hd % W || a.Wa != a.H * a.hd) return hipErrorInvalidValue;
    const int need = (std::max(a.Wa, a.D) / W + 255) / 256;
    switch (need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0) {
      case 1: hipLaunchKernelGGL((norm_fuse_parts<T, 1>), dim3(a.rows), dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((norm_fuse_parts<T, 2>), dim3(a.rows), dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((norm_fuse_parts<T, 4>), dim3(a.rows), dim3(256), 0, s, a); break;
      case 8: hipLaunchKernelGGL((norm_fuse_parts<T, 8>), dim3(a.rows), dim3(256), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
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

// The block's pre-norm: out = g * x / sqrt(mean(x^2) + eps), fp32 statistics.
// WPR waves per row (4 when there are few rows, so a decode batch still
// spreads over the chip); each lane holds up to MAXC W-wide chunks of its
// row in registers, so the row is read once.
template <class T, int WPR, int MAXC>
__global__ void __launch_bounds__(256) rmsnorm_rows(const T *__restrict__ x, const float *__restrict__ g,
                                                    T *__restrict__ out, int rows, int d, float eps) {
  constexpr int W = Vec<T>::W;
  typedef typename Vec<T>::type V;
  __shared__ float part[4];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (4 / WPR) + wave / WPR;
  const int lane = (wave % WPR) * 64 + (threadIdx.x & 63);
  const bool live = row < rows;
  const T *xr = x + (size_t)(live ? row : 0) * d;
  const int nc = d / W;
  V v[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j)   // indices past the row repeat its last chunk
    v[j] = *reinterpret_cast<const V *>(xr + (size_t)min(lane + j * 64 * WPR, nc - 1) * W);
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    float p = 0.0f;
#pragma unroll
    for (int e = 0; e < W; ++e) { const float f = to_f32(v[j][e]); p = fmaf(f, f, p); }
    if (lane + j * 64 * WPR < nc) ss += p;
  }
  ss = wave_sum(ss);
  if (WPR > 1) {
    if ((threadIdx.x & 63) == 0) part[wave] = ss;
    __syncthreads();
    ss = 0.0f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) ss += part[w];
  }
  if (!live) return;
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
  T *o = out + (size_t)row * d;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int c = lane + j * 64 * WPR;
    if (c < nc) {
      V r;
#pragma unroll
      for (int e = 0; e < W; ++e) r[e] = from_f32<T>(g[c * W + e] * to_f32(v[j][e]) * rs);
      *reinterpret_cast<V *>(o + (size_t)c * W) = r;
    }
  }
}

template <class T>
hipError_t launch_rmsnorm(const T *x, const float *g, T *out, int rows, int d, float eps,
                          hipStream_t s) {
  constexpr int W = Vec<T>::W;
  constexpr int MAXC = 8;
  if (d % W || rows <= 0) return hipErrorInvalidValue;
  const int nc = d / W;
  if (rows < 2048 || nc > MAXC * 64) {
    if (nc > MAXC * 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_rows<T, 4, MAXC>), dim3(rows), dim3(256), 0, s, x, g, out, rows, d, eps);
  } else {
    hipLaunchKernelGGL((rmsnorm_rows<T, 1, MAXC>), dim3((rows + 3) / 4), dim3(256), 0, s, x, g, out,
                       rows, d, eps);
  }
  return hipGetLastError();
}
template hipError_t launch_rmsnorm<float>(const float *, const float *, float *, int, int, float, hipStream_t);
template hipError_t launch_rmsnorm<bf16>(const bf16 *, const float *, bf16 *, int, int, float, hipStream_t);

}  // namespace hh

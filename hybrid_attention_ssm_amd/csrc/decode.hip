// One-token decode of the hybrid-head layer.
//
// Attention (Hymba paper §2.1 Eq. (1); meta K/V precomputed and pinned, §2.3
// and App. D; KV-sharing groups and the always-visible meta tokens of the
// authors' replies): the new token at real position p attends to all meta
// keys and to the cached positions max(0, p-W+1)..p (global: 0..p).  Position
// q lives in slot q % cap of a ring cache or slot q of a linear one.  The key
// range is split across workgroups (each keeps a running max, sum and
// weighted V sum per head in the log2 domain) and a second kernel merges the
// splits.  One workgroup serves every query head of its KV head, so each
// cached K/V row is read once per step.
//
// SSM (paper §2.1 Eq. (2)): one recurrence step per channel from the stored
// state and conv history, updated in place.
#include "hh_internal.h"

namespace hh {

namespace {
constexpr int DSPLIT = 512;   // virtual keys per split
constexpr int DTHREADS = 256;

template <class T> struct KV8;
template <> struct KV8<bf16> {
  __device__ static void load(const bf16 *p, float out[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
  }
};
template <> struct KV8<float> {
  __device__ static void load(const float *p, float out[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

__device__ __forceinline__ void merge(float &m, float &l, float *acc, float m2, float l2,
                                      const float *acc2, int n) {
  const float M = fmaxf(m, m2);
  const float s1 = (m == -INFINITY) ? 0.0f : exp2_fast(m - M);
  const float s2 = (m2 == -INFINITY) ? 0.0f : exp2_fast(m2 - M);
  l = l * s1 + l2 * s2;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * s1 + acc2[i] * s2;
  m = M;
}
}  // namespace

// grid (nsplit, G, B); DTHREADS threads; DL = hd/8 lanes per key
template <class T, int HPG>
__global__ void __launch_bounds__(DTHREADS) decode_attn_split(DecodeAttnArgs a) {
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int hd = a.hd, DL = hd / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = tid / DL, sub = tid % DL;
  const int NG = DTHREADS / DL;
  int p = a.len[b] - (a.producer ? 0 : 1);
  const int lo = a.is_global ? 0 : max(0, p - a.window + 1);
  int last = p;
  if (!a.is_ring) last = min(p, a.cap - 1);
  const int L = max(0, last - lo + 1);
  const int nv = a.m + L;
  const int v0 = sp * a.split, v1 = min(nv, v0 + a.split);

  const T *Q = reinterpret_cast<const T *>(a.q) + (size_t)b * a.H * hd;
  const float sl2 = kLog2e / sqrtf((float)hd);
  float q[HPG][8];
#pragma unroll
  for (int hh = 0; hh < HPG; ++hh) {
    float t[8];
    KV8<T>::load(Q + (size_t)(g * HPG + hh) * hd + sub * 8, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[hh][i] = t[i] * sl2;
  }
  float m[HPG], l[HPG], acc[HPG][8];
#pragma unroll
  for (int hh = 0; hh < HPG; ++hh) {
    m[hh] = -INFINITY; l[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[hh][i] = 0.0f;
  }
  const T *Kc = reinterpret_cast<const T *>(a.cache_k) + (size_t)(b * a.G + g) * a.cap * hd;
  const T *Vc = reinterpret_cast<const T *>(a.cache_v) + (size_t)(b * a.G + g) * a.cap * hd;
  const T *Km = reinterpret_cast<const T *>(a.mk) + (size_t)g * a.m * hd;
  const T *Vm = reinterpret_cast<const T *>(a.mv) + (size_t)g * a.m * hd;
  for (int j = v0 + grp; j < v1; j += NG) {
    const T *kp, *vp;
    if (j < a.m) { kp = Km + (size_t)j * hd; vp = Vm + (size_t)j * hd; }
    else {
      const int pos = lo + (j - a.m);
      const int slot = a.is_ring ? pos % a.cap : pos;
      kp = Kc + (size_t)slot * hd; vp = Vc + (size_t)slot * hd;
    }
    float kv[8], vv[8];
    KV8<T>::load(kp + sub * 8, kv);
    KV8<T>::load(vp + sub * 8, vv);
#pragma unroll
    for (int hh = 0; hh < HPG; ++hh) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(q[hh][i], kv[i], s);
      for (int off = 1; off < DL; off <<= 1) s += __shfl_xor(s, off);
      const float mn = fmaxf(m[hh], s);
      const float al = exp2_fast(m[hh] - mn);
      const float pw = exp2_fast(s - mn);
      l[hh] = l[hh] * al + pw;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[hh][i] = fmaf(acc[hh][i], al, pw * vv[i]);
      m[hh] = mn;
    }
  }
  // merge the key groups of this wave (lanes with equal `sub`)
  for (int off = DL; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HPG; ++hh) {
      float acc2[8];
      const float m2 = __shfl_xor(m[hh], off), l2 = __shfl_xor(l[hh], off);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc2[i] = __shfl_xor(acc[hh][i], off);
      merge(m[hh], l[hh], acc[hh], m2, l2, acc2, 8);
    }
  }
  // merge the 4 waves through LDS
  __shared__ float sm[4][HPG], sl[4][HPG], sacc[4][HPG][64];
  if (lane < DL) {
#pragma unroll
    for (int hh = 0; hh < HPG; ++hh) {
      if (lane == 0) { sm[wave][hh] = m[hh]; sl[wave][hh] = l[hh]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) sacc[wave][hh][sub * 8 + i] = acc[hh][i];
    }
  }
  __syncthreads();
  const int stride = hd + 2;
  float *out = a.part + (((size_t)b * a.H + g * HPG) * a.nsplit + sp) * stride;
  for (int it = tid; it < HPG * hd; it += DTHREADS) {
    const int hh = it / hd, d = it % hd;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][hh]);
    float Ls = 0.0f, As = 0.0f;
    for (int w = 0; w < 4; ++w) {
      const float sc = (sm[w][hh] == -INFINITY) ? 0.0f : exp2_fast(sm[w][hh] - M);
      Ls += sl[w][hh] * sc;
      As += sacc[w][hh][d] * sc;
    }
    float *o = out + (size_t)hh * a.nsplit * stride;
    o[2 + d] = As;
    if (d == 0) { o[0] = M; o[1] = Ls; }
  }
}

// grid (B*H); hd threads
template <class T>
__global__ void __launch_bounds__(64) decode_attn_combine(DecodeAttnArgs a) {
  const int bh = blockIdx.x, d = threadIdx.x;
  if (d >= a.hd) return;
  const int stride = a.hd + 2;
  const float *pp = a.part + (size_t)bh * a.nsplit * stride;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pp[(size_t)s * stride]);
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = pp[(size_t)s * stride];
    const float sc = (ms == -INFINITY) ? 0.0f : exp2_fast(ms - M);
    L += pp[(size_t)s * stride + 1] * sc;
    acc += pp[(size_t)s * stride + 2 + d] * sc;
  }
  reinterpret_cast<T *>(a.o)[(size_t)bh * a.hd + d] = from_f32<T>(acc / L);
}

size_t decode_attn_part_bytes(int B, int H, int hd, int m, int max_real, int * /*unused*/,
                              int *nsplit_out) {
  const int nsplit = std::max(1, (m + max_real + DSPLIT - 1) / DSPLIT);
  if (nsplit_out) *nsplit_out = nsplit;
  return (size_t)B * H * nsplit * (hd + 2) * sizeof(float);
}

template <class T>
hipError_t launch_decode_attention(const DecodeAttnArgs &a0, hipStream_t s) {
  DecodeAttnArgs a = a0;
  a.split = DSPLIT;
  const int hpg = a.H / a.G;
  dim3 grid(a.nsplit, a.G, a.B);
  switch (hpg) {
#define HH_DEC_CASE(W) \
    case W: hipLaunchKernelGGL((decode_attn_split<T, W>), grid, dim3(DTHREADS), 0, s, a); break;
    HH_DEC_CASE(1) HH_DEC_CASE(2) HH_DEC_CASE(3) HH_DEC_CASE(4)
    HH_DEC_CASE(5) HH_DEC_CASE(6) HH_DEC_CASE(7) HH_DEC_CASE(8)
#undef HH_DEC_CASE
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(decode_attn_combine<T>, dim3(a.B * a.H), dim3(64), 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_decode_attention<float>(const DecodeAttnArgs &, hipStream_t);
template hipError_t launch_decode_attention<bf16>(const DecodeAttnArgs &, hipStream_t);

// ---------------------------------------------------------------------------
// one SSM step per (sequence, channel)
// ---------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(256) decode_ssm_step(DecodeSsmArgs a) {
  constexpr int NS = 16;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.B * a.D) return;
  const int b = (int)(idx / a.D), c = (int)(idx % a.D);
  const T *z = reinterpret_cast<const T *>(a.z);
  float *conv = a.conv + (size_t)b * (a.k - 1) * a.D;
  const float x = a.xs[idx];
  // window: conv rows (oldest first) then the current xs; tap j multiplies window[j]
  float cv = a.conv_b[c];
  float win[4];
  for (int j = 0; j < a.k - 1; ++j) win[j] = conv[(size_t)j * a.D + c];
  win[a.k - 1] = x;
  for (int j = 0; j < a.k; ++j) cv = fmaf(a.conv_w[(size_t)c * a.k + j], win[j], cv);
  const float u = silu_f(cv);
  const float dt = a.dt[idx];
  const float du = dt * u;
  const float *bc = a.bc + (size_t)b * 2 * NS;
  float *hp = a.h + idx * NS;
  float h[NS];
#pragma unroll
  for (int s = 0; s < NS; s += 4) {
    const float4 v = *reinterpret_cast<const float4 *>(hp + s);
    h[s] = v.x; h[s + 1] = v.y; h[s + 2] = v.z; h[s + 3] = v.w;
  }
  float y = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float A2 = a.A[(size_t)c * NS + s] * kLog2e;
    h[s] = fmaf(exp2_fast(dt * A2), h[s], du * bc[s]);
    y = fmaf(bc[NS + s], h[s], y);
  }
#pragma unroll
  for (int s = 0; s < NS; s += 4)
    *reinterpret_cast<float4 *>(hp + s) = make_float4(h[s], h[s + 1], h[s + 2], h[s + 3]);
  for (int j = 0; j < a.k - 1; ++j) conv[(size_t)j * a.D + c] = win[j + 1];
  reinterpret_cast<T *>(a.y)[idx] = from_f32<T>(y * silu_f(to_f32(z[idx])));
}

template <class T>
hipError_t launch_decode_ssm(const DecodeSsmArgs &a, hipStream_t s) {
  const long n = (long)a.B * a.D;
  hipLaunchKernelGGL(decode_ssm_step<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_decode_ssm<float>(const DecodeSsmArgs &, hipStream_t);
template hipError_t launch_decode_ssm<bf16>(const DecodeSsmArgs &, hipStream_t);

// ---------------------------------------------------------------------------
// cache length bookkeeping
// ---------------------------------------------------------------------------
__global__ void set_len_kernel(int32_t *len, int B, int value) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B) len[i] = value;
}
__global__ void bump_len_kernel(int32_t *len, int B, int cap, int is_ring) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B && (is_ring || len[i] < cap)) len[i] += 1;
}
hipError_t launch_set_len(int32_t *len, int B, int value, hipStream_t s) {
  hipLaunchKernelGGL(set_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, B, value);
  return hipGetLastError();
}
hipError_t launch_bump_len(int32_t *len, int B, int cap, int is_ring, hipStream_t s) {
  hipLaunchKernelGGL(bump_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, B, cap, is_ring);
  return hipGetLastError();
}

}  // namespace hh

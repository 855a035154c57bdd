// Attention heads of the hybrid-head layer, prefill
// (Hymba paper §2.1 Eq. (1) with the 1/sqrt(d) scale of the authors' reply;
// meta tokens always visible plus a causal sliding window, the "A-shape" mask
// of the authors' reply on implementation details; global causal attention in
// the global layers, §2.2; grouped-query heads, Table 11 query groups).
//
// Query row at real position i sees every meta key and the real keys j with
// i - W < j <= i (sliding window) or j <= i (global).
//
// bf16 path (head_dim 64): one workgroup per (sequence, KV head, 32 queries);
// wave w handles query head g*(H/G)+w for those 32 queries, so each K/V tile
// staged in LDS serves every head of the group.  Scores are computed
// transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), which leaves one query
// per lane column: the online-softmax statistics are per-lane scalars and the
// probabilities are already in the B-operand layout of O^T = V^T P^T.  V is
// transposed into LDS as it is staged.  Only the key tiles that intersect the
// window band (plus the meta tiles) are visited; masking is applied only on
// tiles that cross a boundary.
//
// fp32 path: one wavefront per (query, head), lanes over head_dim, exact
// online softmax in fp32.
#include "hh_internal.h"

namespace hh {

namespace {

constexpr int HD = 64;      // bf16 path head dim
constexpr int BQ = 32;      // queries per workgroup
constexpr int BKV = 64;     // keys per tile
constexpr int TILE_CHUNKS = BKV * HD / 8;   // 16-byte chunks per K (or V) tile

__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }

__device__ __forceinline__ float wave_max32(float v) {  // combine lane l and l^32
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum32(float v) { return v + __shfl_xor(v, 32); }

}  // namespace

template <int NW>
__global__ void __launch_bounds__(NW * 64)
attn_prefill_bf16(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int K_PER_T = (TILE_CHUNKS + NT - 1) / NT;
  constexpr int V_PER_T = (256 + NT - 1) / NT;
  __shared__ uint4 sK[2][TILE_CHUNKS];
  __shared__ uint4 sVt[2][TILE_CHUNKS];

  const int hpg = NW;
  const int nqt = (a.n + BQ - 1) / BQ;
  const int qt = nqt - 1 - (int)blockIdx.x;  // heaviest (latest) query tiles first
  const int g = blockIdx.y, b = blockIdx.z;
  const int q0 = qt * BQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int h = g * hpg + wave;
  const int qpos = q0 + lr;                 // this lane's query (column)
  const bf16 *Q = reinterpret_cast<const bf16 *>(a.q);
  const bf16 *Kr = reinterpret_cast<const bf16 *>(a.k) + (size_t)(b * a.G + g) * a.n * HD;
  const bf16 *Vr = reinterpret_cast<const bf16 *>(a.v) + (size_t)(b * a.G + g) * a.n * HD;
  const bf16 *Km = reinterpret_cast<const bf16 *>(a.mk) + (size_t)g * a.m * HD;
  const bf16 *Vm = reinterpret_cast<const bf16 *>(a.mv) + (size_t)g * a.m * HD;
  const int Wa = a.H * HD;

  // Q^T fragments (B operand of S^T = K Q^T): lane holds query lr, dims 16kk+8lh..+7
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qpos < a.n)
      v = *reinterpret_cast<const uint4 *>(Q + ((size_t)b * a.n + qpos) * Wa + h * HD + kk * 16 + lh * 8);
    qf[kk] = __builtin_bit_cast(bf16x8, v);
  }

  // tile schedule: meta tiles, then the real tiles meeting [q0-W+1, q0+BQ-1]
  const int n_meta_t = (a.m + BKV - 1) / BKV;
  const int qlast = min(q0 + BQ - 1, a.n - 1);
  const int lo_pos = a.is_global ? 0 : max(0, q0 - a.window + 1);
  const int t_lo = lo_pos / BKV, t_hi = qlast / BKV;
  const int n_tiles = n_meta_t + (t_hi - t_lo + 1);

  // staging registers
  uint4 rk[K_PER_T];
  uint4 rv[V_PER_T][2];
  auto tile_info = [&](int t, const bf16 *&Kp, const bf16 *&Vp, int &kbase, int &klim, bool &meta) {
    if (t < n_meta_t) { meta = true; kbase = t * BKV; klim = a.m; Kp = Km; Vp = Vm; }
    else { meta = false; kbase = (t_lo + t - n_meta_t) * BKV; klim = a.n; Kp = Kr; Vp = Vr; }
  };
  auto gload = [&](int t) {
    const bf16 *Kp, *Vp; int kbase, klim; bool meta;
    tile_info(t, Kp, Vp, kbase, klim, meta);
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3, dc = c & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < TILE_CHUNKS && kbase + r < klim)
        v = *reinterpret_cast<const uint4 *>(Kp + (size_t)(kbase + r) * HD + dc * 8);
      rk[i] = v;
    }
    // V: item = (key pair kp, d-chunk dc); 256 items
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int it = tid + i * NT;
      const int kp = it >> 3, dc = it & 7;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (it < 256) {
        const int k0 = kbase + 2 * kp;
        if (k0 < klim) v0 = *reinterpret_cast<const uint4 *>(Vp + (size_t)k0 * HD + dc * 8);
        if (k0 + 1 < klim) v1 = *reinterpret_cast<const uint4 *>(Vp + (size_t)(k0 + 1) * HD + dc * 8);
      }
      rv[i][0] = v0;
      rv[i][1] = v1;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < TILE_CHUNKS) sK[buf][swz(c >> 3, c & 7)] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int it = tid + i * NT;
      if (it < 256) {
        const int kp = it >> 3, dc = it & 7;
        const unsigned short *e0 = reinterpret_cast<const unsigned short *>(&rv[i][0]);
        const unsigned short *e1 = reinterpret_cast<const unsigned short *>(&rv[i][1]);
        // Vt row d = 8dc+j holds keys; pair (2kp, 2kp+1) is 4 bytes in chunk kp/4
        char *base = reinterpret_cast<char *>(sVt[buf]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = dc * 8 + j;
          const unsigned int pair = (unsigned int)e0[j] | ((unsigned int)e1[j] << 16);
          *reinterpret_cast<unsigned int *>(base + swz(d, kp >> 2) * 16 + (kp & 3) * 4) = pair;
        }
      }
    }
  };

  const float sl2 = kLog2e * rsqrtf((float)HD);
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { o[0][r] = 0.0f; o[1][r] = 0.0f; }

  gload(0);
  sstore(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const bool more = t + 1 < n_tiles;
    if (more) gload(t + 1);
    const int buf = t & 1;
    const bf16 *Kp, *Vp; int kbase, klim; bool meta;
    tile_info(t, Kp, Vp, kbase, klim, meta);

    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[blk][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, sK[buf][swz(blk * 32 + lr, kk * 2 + lh)]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[blk], 0, 0, 0);
      }
    }
    // does this tile cross a boundary for this wave's queries?
    bool need_mask;
    if (meta) need_mask = kbase + BKV > a.m;
    else need_mask = (kbase + BKV - 1 > q0) || (kbase + BKV > a.n) ||
                     (!a.is_global && kbase < q0 + BQ - 1 - a.window + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[blk][r] * sl2;
        if (need_mask) {
          const int key = kbase + blk * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          bool ok;
          if (meta) ok = key < a.m;
          else ok = key < a.n && key <= qpos && (a.is_global || qpos - key < a.window);
          x = ok ? x : -INFINITY;
        }
        s[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(s[blk][r] - m_use);
        s[blk][r] = p;
        rs += p;
      }
    rs = wave_sum32(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) { o[0][r] *= alpha; o[1][r] *= alpha; }
    // O^T += V^T P^T over the 64 keys, 16 per MFMA
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)s[ks >> 1][8 * (ks & 1) + e];
      const char *vb = reinterpret_cast<const char *>(sVt[buf]);
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk) {
        const int d = dblk * 32 + lr;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vb + swz(d, 2 * ks) * 16 + lh * 8);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vb + swz(d, 2 * ks + 1) * 16 + lh * 8);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dblk], 0, 0, 0);
      }
    }
    if (more) sstore((t + 1) & 1);
    __syncthreads();
  }

  if (qpos < a.n) {
    const float inv = 1.0f / l_run;
    bf16 *O = reinterpret_cast<bf16 *>(a.o) + ((size_t)b * a.n + qpos) * Wa + h * HD;
#pragma unroll
    for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[dblk][4 * j + e] * inv);
        *reinterpret_cast<bf16x4 *>(O + dblk * 32 + 8 * j + 4 * lh) = w;
      }
  }
}

// fp32: one wave per (query, head, sequence); lanes over head_dim (<= 64)
__global__ void __launch_bounds__(256)
attn_prefill_f32(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int total = a.B * a.n * a.H;
  if (wid >= total) return;
  const int h = wid % a.H;
  const int qpos = (wid / a.H) % a.n;
  const int b = wid / (a.H * a.n);
  const int g = h / (a.H / a.G);
  const int hd = a.hd;
  const int Wa = a.H * hd;
  const float *Q = reinterpret_cast<const float *>(a.q) + ((size_t)b * a.n + qpos) * Wa + h * hd;
  const float *Kr = reinterpret_cast<const float *>(a.k) + (size_t)(b * a.G + g) * a.n * hd;
  const float *Vr = reinterpret_cast<const float *>(a.v) + (size_t)(b * a.G + g) * a.n * hd;
  const float *Km = reinterpret_cast<const float *>(a.mk) + (size_t)g * a.m * hd;
  const float *Vm = reinterpret_cast<const float *>(a.mv) + (size_t)g * a.m * hd;
  const bool act = lane < hd;
  const float q = act ? Q[lane] : 0.0f;
  const float scale = 1.0f / sqrtf((float)hd);
  float m_run = -INFINITY, l_run = 0.0f, acc = 0.0f;
  const int lo = a.is_global ? 0 : max(0, qpos - a.window + 1);
  const int nkeys = a.m + (qpos - lo + 1);
  for (int j = 0; j < nkeys; ++j) {
    const float *kp, *vp;
    if (j < a.m) { kp = Km + (size_t)j * hd; vp = Vm + (size_t)j * hd; }
    else { const int pos = lo + (j - a.m); kp = Kr + (size_t)pos * hd; vp = Vr + (size_t)pos * hd; }
    float s = act ? q * kp[lane] : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    s *= scale;
    const float m_new = fmaxf(m_run, s);
    const float alpha = expf(m_run - m_new);
    const float p = expf(s - m_new);
    l_run = l_run * alpha + p;
    acc = acc * alpha + (act ? p * vp[lane] : 0.0f);
    m_run = m_new;
  }
  if (act) reinterpret_cast<float *>(a.o)[((size_t)b * a.n + qpos) * Wa + h * hd + lane] = acc / l_run;
}

template <>
hipError_t launch_attention<bf16>(const AttnArgs &a, hipStream_t s) {
  const int hpg = a.H / a.G;
  dim3 grid((a.n + BQ - 1) / BQ, a.G, a.B);
  switch (hpg) {
#define HH_ATTN_CASE(W) \
    case W: hipLaunchKernelGGL(attn_prefill_bf16<W>, grid, dim3(W * 64), 0, s, a); break;
    HH_ATTN_CASE(1) HH_ATTN_CASE(2) HH_ATTN_CASE(3) HH_ATTN_CASE(4)
    HH_ATTN_CASE(5) HH_ATTN_CASE(6) HH_ATTN_CASE(7) HH_ATTN_CASE(8)
#undef HH_ATTN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_attention<float>(const AttnArgs &a, hipStream_t s) {
  const long waves = (long)a.B * a.n * a.H;
  dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL(attn_prefill_f32, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hh

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
// probabilities are already in the B-operand layout of O^T = V^T P^T.  V^T
// fragments come from transposing LDS reads.  Only the key tiles that intersect the
// window band (plus the meta tiles) are visited; masking is applied only on
// tiles that cross a boundary.
//
// fp32 path: one wavefront per (query, head), lanes over head_dim, exact
// online softmax in fp32.
#include "attn_dev.h"

namespace hh {

using namespace adev;

template <int NW>
// 4 waves per SIMD (at most 128 VGPRs): three 48 KB workgroups per CU
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
attn_prefill_bf16(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ uint4 sK0[TILE_UNITS], sK1[TILE_UNITS], sK2[TILE_UNITS];
  __shared__ uint4 sV0[TILE_UNITS], sV1[TILE_UNITS], sV2[TILE_UNITS];
  __shared__ float sq_part[NW][32];   // fused norm: each head's O^2 sums per query
  __shared__ float sbeta[NW * HD];     // fused norm: the group's betas
  const int bx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
#include "attn_body.inc"
#endif
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

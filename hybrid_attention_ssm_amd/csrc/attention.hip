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
#include "hh_internal.h"

namespace hh {

namespace {

constexpr int HD = 64;      // bf16 path head dim
constexpr int BQ = 32;      // queries per workgroup
constexpr int BKV = 64;     // keys per tile

// 16-byte chunk c of K/V tile row `row` sits at slot c ^ slot_xor(row).  The
// LDS serves 256 bytes (64 banks) per cycle.  K fragment reads take 16 rows
// per cycle, two rows per 256 bytes, so the eight even rows and the eight odd
// rows need distinct slots: slot_xor is a permutation of (row/2) % 8.  The
// transposing V reads take 4 consecutive rows x 32 bytes per 16 lanes, so the
// two rows of a 4-row group that share a 256-byte half (r, r + 2) must differ
// in the slot's bit 2, which the permutation (j%2)*4 + j/2 of j = (row/2) % 8
// also gives.  Both read patterns are then free of bank conflicts.
__device__ __forceinline__ int slot_xor(int row) {
  const int j = (row >> 1) & 7;
  return ((j & 1) << 2) | (j >> 1);
}
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ slot_xor(row)); }

// combine lane l with lane l ^ 32 (v_permlane32_swap: the two half-waves
// trade values in the VALU, no LDS round trip)
__device__ __forceinline__ float other_half(float v, bool low) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // r[0]: lanes 0-31 keep v, lanes 32-63 get v of lane l-32; r[1]: lanes 0-31
  // get v of lane l+32, lanes 32-63 keep v
  return __uint_as_float(low ? r[1] : r[0]);
}
__device__ __forceinline__ float wave_max32(float v, bool low) { return fmaxf(v, other_half(v, low)); }
__device__ __forceinline__ float wave_sum32(float v, bool low) { return v + other_half(v, low); }

}  // namespace

// K and V tiles are streamed into LDS as they lie in memory (64 keys x 128 B,
// 16-byte chunks XOR-swizzled per row) by buffer_load ... lds, STAGES tiles
// deep.  The V^T operand of O^T = V^T P^T is read with ds_read_b64_tr_b16:
// inside each 16-lane group, lane j receives element j%4 of the 8-byte loads
// addressed by lanes 4k + j/4 (k = 0..3), so lane l addressing key row
// 16ks + 4(l/32) + (l%16)/4 (+8) and columns 32dblk + 16((l/16)%2) + 4(l%4)
// hands every lane the 4 consecutive keys of its own d = 32dblk + l%32.
constexpr int ASTAGES = 3;
constexpr int TILE_UNITS = BKV * HD / 8;     // 512 16-byte units per K (or V) tile

template <int NW>
// 4 waves per SIMD (at most 128 VGPRs): three 48 KB workgroups per CU
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
attn_prefill_bf16(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  // one LDS array per stage: reads of one stage then provably do not alias the
  // DMA into another, so the compiler waits only for the tile being read
  __shared__ uint4 sK0[TILE_UNITS], sK1[TILE_UNITS], sK2[TILE_UNITS];
  __shared__ uint4 sV0[TILE_UNITS], sV1[TILE_UNITS], sV2[TILE_UNITS];
  __shared__ float sq_part[NW][32];   // fused norm: each head's O^2 sums per query
  __shared__ float sbeta[NW * HD];     // fused norm: the group's betas
  static_assert(ASTAGES == 3, "three stage arrays");

  const int nqt = (a.n + BQ - 1) / BQ;
  const int qt = nqt - 1 - (int)blockIdx.x;  // heaviest (latest) query tiles first
  const int g = blockIdx.y, b = blockIdx.z;
  const int q0 = qt * BQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lr = lane & 31, lh = lane >> 5;
  const int h = g * NW + wave;
  const int qpos = q0 + lr;
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

  const int n_meta_t = (a.m + BKV - 1) / BKV;
  const int qlast = min(q0 + BQ - 1, a.n - 1);
  const int lo_pos = a.is_global ? 0 : max(0, q0 - a.window + 1);
  const int t_lo = lo_pos / BKV, t_hi = qlast / BKV;
  const int n_tiles = n_meta_t + (t_hi - t_lo + 1);

  // DMA: per stage 8 wave-instructions of 64 x 16 bytes fill the K tile and 8
  // the V tile; each of the min(NW, 4) loader waves issues KI of each (when
  // 8 is not a multiple of the loader count, the extra instructions repeat
  // earlier ones: same bytes to the same slots).  Unit u of a tile is row
  // u/8, slot u%8, holding global chunk slot^((row/2)%8).
  constexpr int LOADERS = NW < 4 ? NW : 4;
  constexpr int KI = (8 + LOADERS - 1) / LOADERS;
  constexpr int INS = 2 * KI;
  typedef __attribute__((address_space(3))) void lds_void;
  const bool loader = wave < LOADERS;
  int voff[KI], part[KI];
#pragma unroll
  for (int j = 0; j < KI; ++j) {
    part[j] = (wave * KI + j) & 7;
    const int u = part[j] * 64 + lane;
    const int row = u >> 3, c = (u & 7) ^ slot_xor(row);
    voff[j] = row * HD * 2 + c * 16;
  }
  auto issue = [&](int t, uint4 *dK, uint4 *dV) {
    if (!loader) return;
    const bool meta = t < n_meta_t;
    const int kbase = meta ? t * BKV : (t_lo + t - n_meta_t) * BKV;
    const int bytes = (meta ? a.m : a.n) * HD * 2;
    // buffers end at the last valid key row: rows past it read as zero
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)(meta ? Km : Kr), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void *)(meta ? Vm : Vr), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < KI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dK + part[j] * 64), 16, voff[j],
                                               kbase * HD * 2, 0, 0);
#pragma unroll
    for (int j = 0; j < KI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dV + part[j] * 64), 16, voff[j],
                                               kbase * HD * 2, 0, 0);
  };
  // ds_read_b64_tr_b16 source offsets (bytes) inside a V tile for
  // (dblk, ks, call): row 16ks + 8call + r0 and column 32dblk + c0 with
  // r0 = 4lh + (l%16)/4 < 8 and c0 = 16((l/16)%2) + 4(l%4) < 32.  slot_xor
  // depends on (row/2) % 8 only, which 16ks leaves alone, so each offset is
  // one of four per-lane bases (call, dblk) plus 2048ks, a constant the read
  // encodes.
  const int tr_row0 = 4 * lh + ((lane & 15) >> 2);
  const int tr_col0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tr_base[2][2];
#pragma unroll
  for (int call = 0; call < 2; ++call)
#pragma unroll
    for (int dblk = 0; dblk < 2; ++dblk) {
      const int row = 8 * call + tr_row0, col = 32 * dblk + tr_col0;
      tr_base[call][dblk] = row * 128 + (((col >> 3) ^ slot_xor(row)) << 4) + (col & 7) * 2;
    }

  const float sl2 = kLog2e * rsqrtf((float)HD);
  // Online softmax with a lazily updated maximum: probabilities are taken as
  // 2^(s*sl2 - m_run) and m_run (with the O rescale) only moves when some
  // lane's tile maximum exceeds it by more than 2^8, so most tiles skip the
  // rescale; the probabilities stay below 2^8 and the result is unchanged.
  constexpr float kLazy = 8.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { o[0][r] = 0.0f; o[1][r] = 0.0f; }

  auto body = [&](int t, const uint4 *sK, const uint4 *sV) {
    const bool meta = t < n_meta_t;
    const int kbase = meta ? t * BKV : (t_lo + t - n_meta_t) * BKV;
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      bf16x8 kf[4];   // a 32-key block's four k-step fragments, read together
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[kk] = __builtin_bit_cast(bf16x8, sK[swz(blk * 32 + lr, kk * 2 + lh)]);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[blk][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s[blk], 0, 0, 0);
    }
    bool need_mask;
    if (meta) need_mask = kbase + BKV > a.m;
    else need_mask = (kbase + BKV - 1 > q0) || (kbase + BKV > a.n) ||
                     (!a.is_global && kbase < q0 + BQ - 1 - a.window + 1);
    if (need_mask) {
      // this lane's query sees keys klo..khi of the tile's source (meta or
      // real); one unsigned range test per score, no per-score branches
      int klo = 0, khi = a.m - 1;
      if (!meta) {
        khi = min(qpos, a.n - 1);
        klo = a.is_global ? 0 : qpos - a.window + 1;
      }
      const bool none = khi < klo;     // only padding lanes past the last query
      const unsigned span = none ? 0u : (unsigned)(khi - klo);
      const int d0 = kbase + 4 * lh - klo;   // key - klo of the lane's first score
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = blk * 32 + 8 * (r >> 2) + (r & 3);
          const bool ok = none ? false : (unsigned)(d0 + off) <= span;
          s[blk][r] = ok ? s[blk][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;   // raw scores: sl2 > 0 keeps the order
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
    mx = wave_max32(mx, lh == 0) * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) { o[0][r] *= alpha; o[1][r] *= alpha; }
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four independent partial sums
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[blk][r], sl2, neg_m));
        s[blk][r] = p;
        rs[r & 3] += p;
      }
    l_run += wave_sum32((rs[0] + rs[1]) + (rs[2] + rs[3]), lh == 0);
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const char *vbase = reinterpret_cast<const char *>(sV);
    bf16x8 pb[4];   // P^T in bf16, all four k-steps, before the V reads
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[ks][e] = (bf16)s[ks >> 1][8 * (ks & 1) + e];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dblk = 0; dblk < 2; ++dblk) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(vbase + tr_base[0][dblk] + 2048 * ks));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(vbase + tr_base[1][dblk] + 2048 * ks));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, both);
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ks], o[dblk], 0, 0, 0);
      }
    }
  };

  const int tlast = n_tiles - 1;
  issue(0, sK0, sV0);
  issue(min(1, tlast), sK1, sV1);
  // the group's betas, read by the epilogue (after a barrier)
  if (a.beta)
    for (int i = tid; i < NW * HD; i += NW * 64) sbeta[i] = a.beta[g * NW * HD + i];
  // tile t lives in stage t % 3; each step waits for its own tile, then (after
  // the barrier frees the stage read one step earlier) issues tile t + 2
#define HH_ATTN_STEP(KC, VC, KN, VN)                                    \
  wait_vmcnt<(ASTAGES - 2) * INS>();                                   \
  __builtin_amdgcn_s_barrier();                                        \
  __builtin_amdgcn_sched_barrier(0);                                   \
  issue(min(t + 2, tlast), KN, VN);                                    \
  body(t, KC, VC);                                                     \
  if (++t >= n_tiles) break;
  for (int t = 0;;) {
    HH_ATTN_STEP(sK0, sV0, sK2, sV2)
    HH_ATTN_STEP(sK1, sV1, sK0, sV0)
    HH_ATTN_STEP(sK2, sV2, sK1, sV1)
  }
#undef HH_ATTN_STEP
  wait_vmcnt<0>();   // the repeated last prefetches, before the workgroup ends

  // lane (lr, lh) holds dims 32dblk + 8j + 4lh + e of query lr.  Under the
  // fused norm the stored value is beta * O and the sum of the unscaled O^2
  // over the group's heads goes to ssq (the row statistics of Eq. (3)).
  float sq = 0.0f;
  if (a.beta) __syncthreads();   // sbeta written
  if (qpos < a.n) {
    const float inv = 1.0f / l_run;
    bf16 *O = reinterpret_cast<bf16 *>(a.o) + ((size_t)b * a.n + qpos) * Wa + h * HD;
#pragma unroll
    for (int dblk = 0; dblk < 2; ++dblk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dblk * 32 + 8 * j + 4 * lh;
        float bt[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (a.beta) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bt[e] = sbeta[wave * HD + d + e];
        }
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = o[dblk][4 * j + e] * inv;
          sq = fmaf(v, v, sq);
          w[e] = (bf16)(bt[e] * v);
        }
        *reinterpret_cast<bf16x4 *>(O + d) = w;
      }
  }
  if (a.ssq) {
    sq = wave_sum32(sq, lh == 0);   // both halves of the query's dims
    if (lh == 0) sq_part[wave][lr] = sq;
    __syncthreads();
    if (wave == 0 && lh == 0 && qpos < a.n) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += sq_part[w][lr];
      a.ssq[((size_t)b * a.n + qpos) * a.G + g] = t;
    }
  }
  if (a.set_len && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = tid; i < a.set_len_n; i += NW * 64) a.set_len[i] = a.set_len_value;
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

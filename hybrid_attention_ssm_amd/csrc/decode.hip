// One-token decode of the hybrid-head layer.
//
// Attention (Hymba paper §2.1 Eq. (1); meta K/V precomputed and pinned, §2.3
// and App. D; KV-sharing groups and the always-visible meta tokens of the
// authors' replies): the new token at real position p attends to all meta
// keys and to the cached positions max(0, p-W+1)..p (global: 0..p).  Position
// q lives in slot q % cap of a ring cache or slot q of a linear one.  The key
// range is split across workgroups (each keeps a running max, sum and
// weighted V sum per head in the log2 domain) and the decode norm merges the
// splits on its way (a single split writes O directly).  One workgroup serves every query head of its KV head, so each
// cached K/V row is read once per step.
//
// SSM (paper §2.1 Eq. (2)): one recurrence step per channel from the stored
// state and conv history, updated in place.
#include <atomic>

#include "hh_internal.h"

namespace hh {

namespace {
constexpr int DSPLIT = 2048;  // most virtual keys per split
constexpr int kNonTemporal = 2;   // cache-policy bits of a buffer load: nt (streaming)
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

// bf16, head_dim 64: MFMA version.  grid (nsplit, G, B), 256 threads.
// Each of the 4 waves walks blocks of 32 keys of the split (block w, w+4, ...):
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = 16 keys, columns = the
//   group's query heads, up to 8 of 16 used), so every lane owns one head;
//   block-wise online softmax in the log2 domain;
//   O^T += V^T P^T, the V block staged in this wave's LDS slice (16-byte
//   chunks XOR-swizzled by row) and read back transposed with
//   ds_read_b64_tr_b16 (lane j of a 16-lane group gets element j%4 of the
//   loads of lanes 4k + j/4).
// The 4 waves' (max, sum, O) are merged through LDS into one partial per
// (sequence, head, split); the decode norm (norm_fuse_parts) merges the
// splits.
constexpr int DB = 32;        // keys per block

template <int HPG>
__global__ void __launch_bounds__(DTHREADS) decode_attn_mfma(DecodeAttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf8;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  constexpr int HD = 64;
  __shared__ uint4 sv[4][DB * HD / 8];                 // 4 KB per wave
  __shared__ float sm[4][16], sl[4][16], so[4][HD][17];
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;          // MFMA column (head), lane group
  const int p = a.len[b] - (a.producer ? 0 : 1);
  const int lo = a.is_global ? 0 : max(0, p - a.window + 1);
  const int last = a.is_ring ? p : min(p, a.cap - 1);
  const int L = max(0, last - lo + 1);
  const int nv = a.m + L;
  const int v0 = sp * a.split, v1 = min(nv, v0 + a.split);
  const bf16 *Kc = reinterpret_cast<const bf16 *>(a.cache_k) + (size_t)(b * a.G + g) * a.cap * HD;
  const bf16 *Vc = reinterpret_cast<const bf16 *>(a.cache_v) + (size_t)(b * a.G + g) * a.cap * HD;
  const bf16 *Km = reinterpret_cast<const bf16 *>(a.mk) + (size_t)g * a.m * HD;
  const bf16 *Vm = reinterpret_cast<const bf16 *>(a.mv) + (size_t)g * a.m * HD;
  // row of virtual key j (meta first, then positions lo..last); callers clamp j
  auto key_row = [&](int j, const bf16 *Mp, const bf16 *Cp) -> const bf16 * {
    if (j < a.m) return Mp + (size_t)j * HD;
    const int pos = lo + (j - a.m);
    const int slot = a.is_ring ? pos % a.cap : pos;
    return Cp + (size_t)slot * HD;
  };

  // Q^T fragments (B operand): lane holds head `col`, dims 32*hh + 8*grp .. +7
  bf8 qf[2];
  {
    const bf16 *Q = reinterpret_cast<const bf16 *>(a.q) + (size_t)b * a.H * HD;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < HPG) v = *reinterpret_cast<const uint4 *>(Q + (size_t)(g * HPG + col) * HD + 32 * hh + 8 * grp);
      qf[hh] = __builtin_bit_cast(bf8, v);
    }
  }
  const float sl2 = kLog2e * 0.125f;   // log2(e) / sqrt(64)
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // ds_read_b64_tr_b16 source offsets in this wave's V slice: (dblk, call)
  int tr_off[8];
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int call = 0; call < 2; ++call) {
      const int row = 16 * call + 4 * grp + (col >> 2);
      const int c16 = 16 * dblk + 4 * (col & 3);
      tr_off[dblk * 2 + call] = row * 128 + ((((c16 >> 3) ^ (row & 7))) << 4) + (c16 & 7) * 2;
    }
  char *vs = reinterpret_cast<char *>(sv[wave]);

  for (int kb0 = v0 + wave * DB; kb0 < v1; kb0 += 4 * DB) {
    const int jmax = v1 - 1;
    // K fragments (A operand of S^T): lane holds key kb0 + 16*kb + col, dims 32*hh + 8*grp
    bf8 kf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16 *kr = key_row(min(kb0 + 16 * kb + col, jmax), Km, Kc);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        kf[kb][hh] = __builtin_bit_cast(bf8, *reinterpret_cast<const uint4 *>(kr + 32 * hh + 8 * grp));
    }
    // V block -> LDS: lane moves 4 chunks: row (q*8 + lane/8), chunk lane%8
    uint4 vv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = q * 8 + (lane >> 3);
      vv[q] = *reinterpret_cast<const uint4 *>(key_row(min(kb0 + row, jmax), Vm, Vc) + 8 * (lane & 7));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = q * 8 + (lane >> 3);
      *reinterpret_cast<uint4 *>(vs + row * 128 + (((lane & 7) ^ (row & 7)) << 4)) = vv[q];
    }
    f32x4 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][hh], qf[hh], st[kb], 0, 0, 0);
    }
    // st[kb][r]: key kb0 + 16*kb + 4*grp + r, head col
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kb0 + 16 * kb + 4 * grp + r;
        const float x = j < v1 ? st[kb][r] * sl2 : -INFINITY;
        st[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float rs = 0.0f;
    bf8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2_fast(st[kb][r] - m_use);
        rs += pr;
        pb[4 * kb + r] = (bf16)pr;
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] *= alpha;
    // P^T's K slots 8*grp + e hold keys 4*grp + e (e < 4) and 16 + 4*grp + e - 4
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
      const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(vs + tr_off[dblk * 2]));
      const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(vs + tr_off[dblk * 2 + 1]));
      const v8i16 both = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      o[dblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, both), pb, o[dblk], 0, 0, 0);
    }
  }
  // o[dblk][r] = O^T[d = 16*dblk + 4*grp + r][head col]; merge the 4 waves
  if (grp == 0) { sm[wave][col] = m_run; sl[wave][col] = l_run; }
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[wave][16 * dblk + 4 * grp + r][col] = o[dblk][r];
  __syncthreads();
  const int stride = HD + 2;
  for (int it = threadIdx.x; it < HPG * HD; it += DTHREADS) {
    const int hh = it / HD, d = it % HD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][hh]);
    float Ls = 0.0f, As = 0.0f;
    for (int w = 0; w < 4; ++w) {
      const float sc = sm[w][hh] == -INFINITY ? 0.0f : exp2_fast(sm[w][hh] - M);
      Ls += sl[w][hh] * sc;
      As += so[w][d][hh] * sc;
    }
    float *out = a.part + (((size_t)b * a.H + g * HPG + hh) * a.nsplit + sp) * stride;
    out[2 + d] = As;
    if (d == 0) { out[0] = M; out[1] = Ls; }
  }
#endif
}

// Same computation with both K and V blocks streamed into LDS by DMA
// (buffer_load_dwordx4 ... lds: full 128-byte rows, no VGPR staging), three
// stages per wave, so a wave's next two blocks are in flight while it works
// on the current one.  The stages are separate LDS arrays and the loop
// rotates through them explicitly: reads of one stage then provably do not
// alias the DMA into another, and the compiler waits only for the block being
// read.  Needs the meta count to be a multiple of the 32-key block so that a
// block is all meta or all cache (one buffer descriptor per block).
// LDS rows are 128 B with 16-byte chunk c of row r stored at chunk c ^ (r % 8).
template <int HPG, int NW>
__device__ __forceinline__ void attn_dma_body(const DecodeAttnArgs &a, int sp, int g, int b) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf8;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int HD = 64;
  constexpr int BLK = DB * HD * 2;          // one K or V block: 4 KB
  constexpr int SLICE = 2 * 2 * BLK;        // per wave: 2 stages of (K, V)
  constexpr int SO = 17;                    // merge-buffer row stride (floats)
  static_assert(NW * HD * SO * 4 <= NW * SLICE / 2, "merge buffer fits the slices");
  __shared__ __attribute__((aligned(16))) char lds0[NW * SLICE / 2];
  __shared__ __attribute__((aligned(16))) char lds1[NW * SLICE / 2];
  __shared__ __attribute__((aligned(16))) char lds2[NW * SLICE / 2];
  __shared__ float sm[NW][16], sl[NW][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int p = a.len[b] - (a.producer ? 0 : 1);
  const int lo = a.is_global ? 0 : max(0, p - a.window + 1);
  const int last = a.is_ring ? p : min(p, a.cap - 1);
  const int L = max(0, last - lo + 1);
  const int nv = a.m + L;
  const int v0 = sp * a.split, v1 = min(nv, v0 + a.split);
  const size_t cache_off = (size_t)(b * a.G + g) * a.cap * HD;
  const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const bf16 *>(a.cache_k) + cache_off), (short)0, a.cap * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const bf16 *>(a.cache_v) + cache_off), (short)0, a.cap * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rkm = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const bf16 *>(a.mk) + (size_t)g * a.m * HD), (short)0, a.m * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvm = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const bf16 *>(a.mv) + (size_t)g * a.m * HD), (short)0, a.m * HD * 2, 0x00020000);
  // real position lo + t sits in slot rbase + t (wrapped once for a ring)
  const int rbase = a.is_ring ? lo % a.cap : lo;
  const int wrap = a.is_ring ? a.cap : 0x7fffffff;
  char *slice0 = lds0 + wave * (SLICE / 2);
  char *slice1 = lds1 + wave * (SLICE / 2);
  char *slice2 = lds2 + wave * (SLICE / 2);
  // DMA of the 32-key block at virtual key kb into stage st: instruction q moves
  // rows 8q .. 8q+7 (lane: row 8q + lane/8, chunk (lane%8) ^ row%8)
  auto issue = [&](int kb, char *kdst) {
    int voff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int j = min(kb + r, v1 - 1);
      int row = j;
      if (kb >= a.m) {   // uniform: the whole block is cache
        row = rbase + (j - a.m);
        row = row >= wrap ? row - wrap : row;
      }
      voff[q] = row * 128 + (((lane & 7) ^ (r & 7)) << 4);
    }
    if (kb < a.m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkm, (lds_void *)(kdst + q * 1024), 16, voff[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvm, (lds_void *)(kdst + BLK + q * 1024), 16, voff[q], 0, 0, 0);
      }
    } else {
      // The cache blocks are streamed (nt): a step reads 1.7 GB of K/V once or
      // twice, far more than the 256 MB last-level cache, and allocating it
      // there evicts the weights and SSM states the step's other kernels
      // reuse.  Measured on the three-layer step: 476 -> 446 us (streaming the
      // window rings too beats caching them for their consumer's second read).
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkc, (lds_void *)(kdst + q * 1024), 16, voff[q], 0, 0, kNonTemporal);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvc, (lds_void *)(kdst + BLK + q * 1024), 16, voff[q], 0, 0,
                                                 kNonTemporal);
      }
    }
  };

  int kb = v0 + wave * DB;
  if (kb < v1) issue(kb, slice0);   // the first block travels with Q
  bf8 qf[2];
  {
    const bf16 *Q = reinterpret_cast<const bf16 *>(a.q) + (size_t)b * a.H * HD;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < HPG) v = *reinterpret_cast<const uint4 *>(Q + (size_t)(g * HPG + col) * HD + 32 * hh + 8 * grp);
      qf[hh] = __builtin_bit_cast(bf8, v);
    }
  }
  const int step = NW * DB;
  if (kb + step < v1) {              // the second block follows Q
    issue(kb + step, slice1);
    wait_vmcnt<8>();                 // Q and the first block have landed
  } else {
    wait_vmcnt<0>();                 // Q (and the first block) have landed
  }
  const float sl2 = kLog2e * 0.125f;   // log2(e) / sqrt(64)
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // K fragment (A operand of S^T): row 16*k2 + col, chunk 4*hh + grp
  int k_off[4];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 16 * k2 + col;
      k_off[k2 * 2 + hh] = r * 128 + (((4 * hh + grp) ^ (r & 7)) << 4);
    }
  // V^T through ds_read_b64_tr_b16 (rows 4*grp + col/4 and 16 + ..., columns 16*dblk + 4*(col%4))
  int tr_off[8];
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int call = 0; call < 2; ++call) {
      const int row = 16 * call + 4 * grp + (col >> 2);
      const int c16 = 16 * dblk + 4 * (col & 3);
      tr_off[dblk * 2 + call] = row * 128 + ((((c16 >> 3) ^ (row & 7))) << 4) + (c16 & 7) * 2;
    }

  auto process = [&](int kb, const char *ks) {
    const char *vs = ks + BLK;
    f32x4 stt[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      stt[k2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf8 kf = __builtin_bit_cast(bf8, *reinterpret_cast<const uint4 *>(ks + k_off[k2 * 2 + hh]));
        stt[k2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[hh], stt[k2], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kb + 16 * k2 + 4 * grp + r;
        const float x = j < v1 ? stt[k2][r] * sl2 : -INFINITY;
        stt[k2][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast(m_run - m_new);
    float rs = 0.0f;
    bf8 pb;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2_fast(stt[k2][r] - m_new);
        rs += pr;
        pb[4 * k2 + r] = (bf16)pr;
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] *= alpha;
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
      const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(vs + tr_off[dblk * 2]));
      const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(vs + tr_off[dblk * 2 + 1]));
      const v8i16 both = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      o[dblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, both), pb, o[dblk], 0, 0, 0);
    }
  };
  if (kb < v1) {
    // Three stages: blocks kb + step and kb + 2 step are in flight while kb is
    // processed.  Past the end nothing is issued, and the wait allows only the
    // blocks that really are in flight (each issue is 8 loads, in order).
    auto refill_wait = [&](int nxt, char *dst) {
      if (nxt < v1) {
        issue(nxt, dst);
        wait_vmcnt<16>();
      } else if (nxt - step < v1) {
        wait_vmcnt<8>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    while (true) {
      refill_wait(kb + 2 * step, slice2);
      process(kb, slice0);
      __builtin_amdgcn_sched_barrier(0);
      kb += step;
      if (kb >= v1) break;
      refill_wait(kb + 2 * step, slice0);
      process(kb, slice1);
      __builtin_amdgcn_sched_barrier(0);
      kb += step;
      if (kb >= v1) break;
      refill_wait(kb + 2 * step, slice1);
      process(kb, slice2);
      __builtin_amdgcn_sched_barrier(0);
      kb += step;
      if (kb >= v1) break;
    }
    wait_vmcnt<0>();
  }
  // merge the 4 waves (the DMA slices become the merge buffer)
  __syncthreads();
  float *so = reinterpret_cast<float *>(lds0);
  if (grp == 0) { sm[wave][col] = m_run; sl[wave][col] = l_run; }
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[(wave * HD + 16 * dblk + 4 * grp + r) * SO + col] = o[dblk][r];
  __syncthreads();
  const int stride = HD + 2;
  for (int it = threadIdx.x; it < HPG * HD; it += NW * 64) {
    const int hh = it / HD, d = it % HD;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w][hh]);
    float Ls = 0.0f, As = 0.0f;
    for (int w = 0; w < NW; ++w) {
      const float sc = sm[w][hh] == -INFINITY ? 0.0f : exp2_fast(sm[w][hh] - M);
      Ls += sl[w][hh] * sc;
      As += so[(w * HD + d) * SO + hh] * sc;
    }
    if (a.nsplit == 1) {   // the only split: this is the output
      reinterpret_cast<bf16 *>(a.o)[((size_t)b * a.H + g * HPG + hh) * HD + d] = (bf16)(As / Ls);
      continue;
    }
    float *out = a.part + (((size_t)b * a.H + g * HPG + hh) * a.nsplit + sp) * stride;
    out[2 + d] = As;
    if (d == 0) { out[0] = M; out[1] = Ls; }
  }
#endif
}

// grid (nsplit, G, B)
template <int HPG, int NW>
__global__ void __launch_bounds__(NW * 64) decode_attn_dma(DecodeAttnArgs a) {
  attn_dma_body<HPG, NW>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Keys per split: a multiple of the 32-key block, at most DSPLIT, and small
// enough that the grid has about kDecodeTargetWG workgroups (a short sliding
// window over few heads would otherwise leave most of the chip idle).  From
// there up to 4 more splits are weighed by (rounds of resident workgroups) x
// (keys per split): the DMA kernel fits kDecodeWGPerCU workgroups on a CU
// (48 KB of LDS each), so a grid that ends in a partial round wastes the
// rest of it.  Batch 128, context 8k: 6 splits (5 full rounds) instead of 7
// (5.8 rounds), global-layer attention 222.6 -> 220.1 us.
constexpr int kDecodeTargetWG = 640;
constexpr int kDecodeWGPerCU = 3;
int device_cus() {
  // queried once per device; concurrent first calls store the same value
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDev) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}
size_t decode_attn_part_bytes(int B, int H, int G, int hd, int m, int max_real, int *split_out,
                              int *nsplit_out) {
  const int nv = std::max(1, m + max_real);
  const long bg = (long)B * G;
  const int want = (int)((kDecodeTargetWG + bg - 1) / bg);
  const int ns_lo = std::max((nv + DSPLIT - 1) / DSPLIT, std::min(want, (nv + 127) / 128));
  const long slots = (long)kDecodeWGPerCU * device_cus();
  int split = 0, nsplit = 0;
  long best = -1;
  for (int ns = ns_lo; ns <= ns_lo + 4; ++ns) {
    const int sp = ((nv + ns - 1) / ns + 31) / 32 * 32;
    const int n = (nv + sp - 1) / sp;
    const long cost = (bg * n + slots - 1) / slots * sp;
    if (best < 0 || cost < best) { best = cost; split = sp; nsplit = n; }
  }
  if (split_out) *split_out = split;
  if (nsplit_out) *nsplit_out = nsplit;
  return (size_t)B * H * nsplit * (hd + 2) * sizeof(float);
}

template <class T>
hipError_t launch_decode_attention(const DecodeAttnArgs &a, hipStream_t s, bool *o_ready) {
  const int hpg = a.H / a.G;
  dim3 grid(a.nsplit, a.G, a.B);
  // the DMA kernel writes O itself when there is a single split; the others
  // always leave per-split partials
  bool direct = false;
  if (sizeof(T) == 2 && a.hd == 64 && a.m % DB == 0 && a.split % DB == 0) {
    // 2-wave workgroups with three 8 KB stages per wave (48 KB, three to a
    // CU).  Against 4-wave workgroups with two stages: the window layer's
    // 640-workgroup grid no longer ends in a partial round (34.9 -> 30.6 us),
    // and the global layer keeps two blocks per wave in flight (231.6 ->
    // 223.2 us at batch 128, context 8k).
    switch (hpg) {
#define HH_DECD_CASE(W) \
      case W: \
        hipLaunchKernelGGL((decode_attn_dma<W, 2>), grid, dim3(128), 0, s, a); \
        break;
      HH_DECD_CASE(1) HH_DECD_CASE(2) HH_DECD_CASE(3) HH_DECD_CASE(4)
      HH_DECD_CASE(5) HH_DECD_CASE(6) HH_DECD_CASE(7) HH_DECD_CASE(8)
#undef HH_DECD_CASE
      default: return hipErrorInvalidValue;
    }
    direct = a.nsplit == 1;
  } else if (sizeof(T) == 2 && a.hd == 64) {
    switch (hpg) {
#define HH_DECM_CASE(W) \
      case W: hipLaunchKernelGGL((decode_attn_mfma<W>), grid, dim3(DTHREADS), 0, s, a); break;
      HH_DECM_CASE(1) HH_DECM_CASE(2) HH_DECM_CASE(3) HH_DECM_CASE(4)
      HH_DECM_CASE(5) HH_DECM_CASE(6) HH_DECM_CASE(7) HH_DECM_CASE(8)
#undef HH_DECM_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (hpg) {
#define HH_DEC_CASE(W) \
      case W: hipLaunchKernelGGL((decode_attn_split<T, W>), grid, dim3(DTHREADS), 0, s, a); break;
      HH_DEC_CASE(1) HH_DEC_CASE(2) HH_DEC_CASE(3) HH_DEC_CASE(4)
      HH_DEC_CASE(5) HH_DEC_CASE(6) HH_DEC_CASE(7) HH_DEC_CASE(8)
#undef HH_DEC_CASE
      default: return hipErrorInvalidValue;
    }
  }
  if (o_ready) *o_ready = direct;
  return hipGetLastError();
}
template hipError_t launch_decode_attention<float>(const DecodeAttnArgs &, hipStream_t, bool *);
template hipError_t launch_decode_attention<bf16>(const DecodeAttnArgs &, hipStream_t, bool *);

// ---------------------------------------------------------------------------
// one SSM step: four lanes per (sequence, channel), four states each, so the
// state, A and B/C move as contiguous 16-byte vectors across the quad.  (A
// producer's len advances in the decode norm, after the step's attention.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float quad_sum(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

// Thread t owns quad t: (sequence, channel) t / 4 and its states 4 (t % 4)
// .. +3.  Every load is independent and issued before any arithmetic; one
// quad per thread at full occupancy keeps the most loads in flight (two or
// four quads per thread measured slower: 15.5 -> 16.7 / 20.2 us).
// SC: Mamba2 heads (Delta per head, one scalar A per head: one exp2 per lane)
template <class T, int K, bool SC>
__global__ void __launch_bounds__(256) decode_ssm_step(DecodeSsmArgs a) {
  constexpr int NS = 16;
  typedef float f32v4 __attribute__((ext_vector_type(4)));
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long idx = t >> 2;                  // sequence * D + channel
  const int q = (int)(t & 3);               // states 4q .. 4q+3
  const bool live = idx < (long)a.B * a.D;
  const long ci = live ? idx : 0;
  const int b = (int)(ci / a.D), c = (int)(ci % a.D);
  float *conv = a.conv + (size_t)b * (K - 1) * a.D + c;
  float win[K], wk[K];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) win[j] = conv[(size_t)j * a.D];   // oldest first
  win[K - 1] = a.xs[ci];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = a.conv_w[(size_t)c * K + j];
  const float cb = a.conv_b[c];
  const int hd_ = SC ? c / (a.D / a.S) : 0;   // Mamba2 head of channel c
  const float dt = SC ? a.dt[(size_t)b * a.S + hd_] : a.dt[ci];
  const float zv = to_f32(reinterpret_cast<const T *>(a.z)[ci]);
  const float4 Bq = *reinterpret_cast<const float4 *>(a.bc + (size_t)b * 2 * NS + 4 * q);
  const float4 Cq = *reinterpret_cast<const float4 *>(a.bc + (size_t)b * 2 * NS + NS + 4 * q);
  const float4 Aq = SC ? make_float4(a.A[hd_], 0.0f, 0.0f, 0.0f)
                       : *reinterpret_cast<const float4 *>(a.A + (size_t)c * NS + 4 * q);
  // The state is read and written once per step, a step's worth of other
  // traffic apart: stream it (nt) rather than let it displace the weights
  // from the last-level cache.
  f32v4 *hp = reinterpret_cast<f32v4 *>(a.h + ci * NS + 4 * q);
  f32v4 h = __builtin_nontemporal_load(hp);
  // tap j multiplies window row j (tap K-1 the current row)
  float cv = cb;
#pragma unroll
  for (int j = 0; j < K; ++j) cv = fmaf(wk[j], win[j], cv);
  const float du = dt * silu_f(cv);
  const float d2 = dt * kLog2e;
  if constexpr (SC) {
    const float decay = exp2_fast(d2 * Aq.x);
    h.x = fmaf(decay, h.x, du * Bq.x);
    h.y = fmaf(decay, h.y, du * Bq.y);
    h.z = fmaf(decay, h.z, du * Bq.z);
    h.w = fmaf(decay, h.w, du * Bq.w);
  } else {
    h.x = fmaf(exp2_fast(d2 * Aq.x), h.x, du * Bq.x);
    h.y = fmaf(exp2_fast(d2 * Aq.y), h.y, du * Bq.y);
    h.z = fmaf(exp2_fast(d2 * Aq.z), h.z, du * Bq.z);
    h.w = fmaf(exp2_fast(d2 * Aq.w), h.w, du * Bq.w);
  }
  float y = Cq.x * h.x;
  y = fmaf(Cq.y, h.y, y);
  y = fmaf(Cq.z, h.z, y);
  y = fmaf(Cq.w, h.w, y);
  y = quad_sum(y);
  if (!live) return;
  __builtin_nontemporal_store(h, hp);
  if (q == 0) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) conv[(size_t)j * a.D] = win[j + 1];
    reinterpret_cast<T *>(a.y)[idx] = from_f32<T>(y * silu_f(zv));
  }
}

template <class T>
hipError_t launch_decode_ssm(const DecodeSsmArgs &a, hipStream_t s) {
  const long n = (long)a.B * a.D * 4;
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool sc = a.S > 0;
  switch (a.k) {
#define HH_SSM_CASE(KK) \
    case KK: \
      if (sc) hipLaunchKernelGGL((decode_ssm_step<T, KK, true>), grid, dim3(256), 0, s, a); \
      else hipLaunchKernelGGL((decode_ssm_step<T, KK, false>), grid, dim3(256), 0, s, a); \
      break;
    HH_SSM_CASE(2) HH_SSM_CASE(3) HH_SSM_CASE(4)
#undef HH_SSM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_decode_ssm<float>(const DecodeSsmArgs &, hipStream_t);
template hipError_t launch_decode_ssm<bf16>(const DecodeSsmArgs &, hipStream_t);

}  // namespace hh

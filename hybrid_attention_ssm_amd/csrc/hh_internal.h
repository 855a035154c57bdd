// Internal declarations shared by the HIP translation units of libhymba_hh.
// Device helpers, the in-projection column map and the kernel launchers that
// hh_api.cpp drives.  Not part of the public ABI (include/hh.h).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace hh {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// round to nearest even (hardware v_cvt on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ---- fast transcendental helpers (fp32) ------------------------------------
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).  gfx9 s_waitcnt immediate: vmcnt[3:0] at
// bits 3:0 and vmcnt[5:4] at 15:14; expcnt and lgkmcnt at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until this wave's LDS (and scalar-memory) operations have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
// x * sigmoid(x) with sigmoid = 1 / (1 + 2^(-x log2 e)); saturates cleanly:
// x -> -inf gives 2^(+inf) = inf, rcp(inf) = 0.
__device__ __forceinline__ float silu_f(float x) {
  return x * rcp_fast(1.0f + exp2_fast(-x * kLog2e));
}
// log(1 + e^v) without overflow: max(v, 0) + log1p(t), t = e^-|v| in (0, 1].
// With u = fl(1 + t) (so u - 1 is exact), log1p(t) = log(u) + log(1 + r) where
// r = (t - (u - 1)) / u is the relative rounding error of 1 + t, |r| <= 2^-24;
// log(1 + r) = r to within r^2 / 2.  1/u (u in [1, 2]) is taken from the chord
// 1.5 - u/2, within 6 %, which only scales the already tiny r.  Two
// transcendentals (2^x, log2) and no division; small t keeps full relative
// accuracy (u = 1 gives exactly t).
__device__ __forceinline__ float softplus_f(float v) {
  constexpr float kLn2 = 0.6931471805599453f;
  const float t = exp2_fast(-fabsf(v) * kLog2e);
  const float u = 1.0f + t;
  const float r = (t - (u - 1.0f)) * fmaf(-0.5f, u, 1.5f);
  return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, r);
}

// ---- the in-projection column map ------------------------------------------
// Columns of P = X W_in^T: Q [0, Wa) | K [Wa, Wa+KV) | V [Wa+KV, Wa+2KV) |
// xs (D) | z (D) | dt (Ddt: D, or one per Mamba2 head) | B (N) | C (N);
// KV = 0 for a consumer layer.
enum EpiMode : int { EPI_PREFILL = 0, EPI_DECODE = 1, EPI_META = 2 };

struct InProjOut {
  int mode;
  int row0;                   // global row of the GEMM's first row (a launch over a row range)
  int Wa, KV, D, N, hd, n_rows_per_seq;  // n_rows_per_seq: seqlen (prefill) or m (meta)
  int Ddt;                    // dt block width: D, or the Mamba2 head count
  void *q;                    // [rows, Wa]
  void *k_full, *v_full;      // prefill: [B, G, n, hd]; meta: [G, m, hd]
  void *cache_k, *cache_v;    // prefill/decode cache [B, G, cap, hd] (may be null)
  int cap, is_ring;
  const int32_t *len;         // decode: position of the new token per row
  // The SSM features: row-major [rows, width] when ssm_rows is 0 (decode),
  // else channel-block-major (ssm_index: blocks of 64 columns, each holding
  // all ssm_rows rows), so that a scan wave's 64 channels are one contiguous
  // 256-byte run per row and its chunk one contiguous stream.
  int ssm_rows;
  float *xs;                  // [rows, D] fp32 (SSM input features)
  void *z;                    // [rows, D]
  float *dt;                  // [rows, Ddt] softplus(dt + bias)
  float *bc;                  // [rows, 2N] B then C
  const float *dt_bias;       // [D]
  // Rotary embedding of Q and K (rope_base 0: none).  Position of a row:
  // meta mode, the row; prefill, rope_m + row % n_rows_per_seq; decode,
  // rope_m + len[row] + len_bias (-1 for a consumer, whose producer has
  // already counted the token).  Pair i turns by pos * rope_f0 * rope_ratio^i
  // revolutions (rope_f0 = 1/(2 pi), rope_ratio = base^(-2/hd), from the host
  // in double).
  float rope_base;
  int rope_m, len_bias;
  double rope_f0, rope_ratio;
};

// How the in-projection's epilogue meets the rotation pairs (dims i and
// i + hd/2 of a Q or K head):
//   ROPE_PAIRED_COLS  the GEMM reads each head's weight rows in pair order
//                     (inproj_src_row), so a group of W columns holds W/2
//                     whole pairs, stored back at their natural columns;
//   ROPE_SPLIT_GROUPS the GEMM hands over two groups at once, dims d..d+W-1
//                     and d+hd/2.. of one head (store_pair): a lane of the
//                     256x256-tile kernel owns exactly these, as its wave's 64
//                     columns are one head.
enum RopeMode : int { ROPE_NONE = 0, ROPE_PAIRED_COLS = 1, ROPE_SPLIT_GROUPS = 2 };

// Weight row feeding output column n under ROPE_PAIRED_COLS: the columns of
// each Q and K head come out in pair order, dims (0, hd/2, 1, hd/2+1, ...).
// Heads never straddle a GEMM tile (Q starts at 0, K at H*hd, tiles are
// multiples of 64 wide).
__device__ __forceinline__ int inproj_src_row(const InProjOut &e, int n) {
  if (n >= e.Wa + e.KV) return n;
  const int j = n % e.hd;
  return n - j + ((j & 1) ? e.hd / 2 : 0) + (j >> 1);
}

// Element (row, col) of an SSM feature array in the channel-block-major
// layout: 64-column blocks, block-major, rows inside a block, the block's
// 64 columns contiguous.  A buffer for `rows` rows and width w holds
// rows * round_up(w, 64) elements.
__host__ __device__ __forceinline__ size_t ssm_index(size_t row, int col, size_t rows) {
  return ((size_t)(col >> 6) * rows + row) * 64 + (col & 63);
}
__device__ __forceinline__ size_t ssm_at(const InProjOut &e, int row, int col, int width) {
  return e.ssm_rows ? ssm_index(row, col, e.ssm_rows) : (size_t)row * width + col;
}

// Store 8 consecutive columns col..col+7 of one row (col % 8 == 0).  Every
// column-block boundary of the map is a multiple of 8, so the 8 values always
// belong to one block and are written with vector stores.
template <class T>
__device__ __forceinline__ void store8_T(T *dst, const float v[8]) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8 *>(dst) = o;
  } else {
    *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Store W (2, 4 or 8) consecutive values (converted to T).
template <class T, int W>
__device__ __forceinline__ void storeW_T(T *dst, const float v[W]) {
  static_assert(W == 2 || W == 4 || W == 8, "group width");
  if constexpr (W == 8) {
    store8_T(dst, v);
  } else if constexpr (W == 2) {
    if constexpr (sizeof(T) == 2) {
      typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
      bf16x2 o;
      o[0] = (bf16)v[0];
      o[1] = (bf16)v[1];
      *reinterpret_cast<bf16x2 *>(dst) = o;
    } else {
      *reinterpret_cast<float2 *>(dst) = make_float2(v[0], v[1]);
    }
  } else if constexpr (sizeof(T) == 2) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x4 *>(dst) = o;
  } else {
    *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Load W (4 or 8) consecutive values as fp32.
template <class T, int W>
__device__ __forceinline__ void loadW_T(const T *src, float v[W]) {
  static_assert(W == 4 || W == 8, "group width");
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((__vector_size__(W * sizeof(__bf16)))) __bf16 bfW;
    const bfW x = *reinterpret_cast<const bfW *>(src);
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = (float)x[i];
  } else {
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const float4 x = reinterpret_cast<const float4 *>(src)[q];
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  }
}

// Column-side part of a group of W consecutive columns (col % W == 0; no
// block boundary inside a group), resolved once per lane: which block of the
// map the columns fall in, the offset inside it and, for the Delta block,
// the biases.
template <int W>
struct ColInfo {
  int seg;       // 0 Q, 1 K, 2 V, 3 xs, 4 z, 5 dt, 6 B|C
  int c;         // column offset inside the block
  int g, d;      // K/V: head and position inside the head
  float bias[W];
  // RoPE (Q, K): pair j of the group turns by pos * f_j revolutions, f_j =
  // base^(-2i/hd) / (2 pi) held as hi + lo floats (i the pair's low dim);
  // W/2 pairs under ROPE_PAIRED_COLS, W under ROPE_SPLIT_GROUPS
  float rf_hi[W], rf_lo[W];
};

template <int W, int ROPE>
__device__ __forceinline__ ColInfo<W> inproj_col(const InProjOut &e, int col) {
  ColInfo<W> ci{};
  const int Wa = e.Wa, KV = e.KV, D = e.D;
  auto rope_freqs = [&](int c) {   // c: column inside the Q or K block
    if constexpr (ROPE != ROPE_NONE) {
      constexpr int NP = ROPE == ROPE_PAIRED_COLS ? W / 2 : W;
      const int i0 = ROPE == ROPE_PAIRED_COLS ? (c % e.hd) >> 1 : c % e.hd;
      double f = e.rope_f0, r = e.rope_ratio;   // f0 * ratio^i0 by squaring
      for (int k = i0; k; k >>= 1, r *= r)
        if (k & 1) f *= r;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        ci.rf_hi[j] = (float)f;
        ci.rf_lo[j] = (float)(f - (double)ci.rf_hi[j]);
        f *= e.rope_ratio;
      }
    }
  };
  if (col < Wa) { ci.seg = 0; ci.c = col; rope_freqs(col); return ci; }
  col -= Wa;
  if (col < 2 * KV) {
    ci.seg = col < KV ? 1 : 2;
    ci.c = col < KV ? col : col - KV;
    ci.g = ci.c / e.hd;
    ci.d = ci.c - ci.g * e.hd;
    if (ci.seg == 1) rope_freqs(ci.c);
    return ci;
  }
  col -= 2 * KV;
  if (col < D) { ci.seg = 3; ci.c = col; return ci; }
  col -= D;
  if (col < D) { ci.seg = 4; ci.c = col; return ci; }
  col -= D;
  if (col < e.Ddt) {
    ci.seg = 5; ci.c = col;
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const float4 bq = *reinterpret_cast<const float4 *>(e.dt_bias + col + 4 * q);
      ci.bias[4 * q] = bq.x; ci.bias[4 * q + 1] = bq.y; ci.bias[4 * q + 2] = bq.z; ci.bias[4 * q + 3] = bq.w;
    }
    return ci;
  }
  ci.seg = 6; ci.c = col - e.Ddt;
  return ci;
}

// sin and cos of 2 pi r for |r| <= 1/2 (and a little beyond): quarter turns
// are split off (x = 4r = q + f, |f| <= 1/2), then the Taylor series of sin
// and cos at t = f pi/2, |t| <= pi/4, through t^9 and t^10 (truncation below
// 2e-9), and the quadrant q turns the pair (selects, no branches).
__device__ __forceinline__ void sincos_rev(float r, float &sn, float &cs) {
  const float x = 4.0f * r;
  const float q = rintf(x);
  const float t = (x - q) * 1.5707963267948966f;
  const float t2 = t * t;
  const float sp = fmaf(t * t2, fmaf(t2, fmaf(t2, fmaf(t2, 2.7557319223985893e-6f, -1.9841269841269841e-4f),
                                              8.3333333333333333e-3f), -1.6666666666666667e-1f), t);
  const float cp = fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, -2.7557319223985888e-7f, 2.4801587301587302e-5f),
                                                   -1.3888888888888889e-3f), 4.1666666666666667e-2f), -0.5f), 1.0f);
  const int qi = (int)q;
  const float s1 = (qi & 1) ? cp : sp, c1 = (qi & 1) ? -sp : cp;
  sn = (qi & 2) ? -s1 : s1;
  cs = (qi & 2) ? -c1 : c1;
}

// Turn the pair (x, y) = (dim i, dim i + hd/2) by pos * f revolutions, f =
// hi + lo.  The angle is reduced in revolutions with the exact product
// pos * hi (plus pos * lo), so only |r| <= 1/2 turn reaches sincos_rev.
__device__ __forceinline__ void rope_pair(float hi, float lo, float p, float &x, float &y) {
  const float a = p * hi;
  const float b = fmaf(p, lo, fmaf(p, hi, -a));
  float sn, cs;
  sincos_rev((a - rintf(a)) + b, sn, cs);
  const float nx = fmaf(x, cs, -y * sn), ny = fmaf(y, cs, x * sn);
  x = nx;
  y = ny;
}

// position of a row of the in-projection for the rotary embedding
__device__ __forceinline__ int rope_position(const InProjOut &e, int row) {
  if (e.mode == EPI_META) return row;
  if (e.mode == EPI_DECODE) return e.rope_m + e.len[row] + e.len_bias;
  return e.rope_m + row % e.n_rows_per_seq;
}

// One row's group of W consecutive columns of the fused projection (see
// ColInfo) to its destination.  Under ROPE_PAIRED_COLS the Q and K groups
// arrive in pair order and are turned here; under ROPE_SPLIT_GROUPS they
// come through inproj_store_pair, already turned.
template <class T, int W, int ROPE>
__device__ __forceinline__ void inproj_storeW(const InProjOut &e, int row, const ColInfo<W> &ci,
                                              const float v[W]) {
  const int Wa = e.Wa, D = e.D;
  // turn the group's W/2 pairs (in pair order) into low and high dims
  auto turn = [&](float lo[W / 2], float hi[W / 2]) {
    const float p = (float)rope_position(e, row);
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      lo[j] = v[2 * j];
      hi[j] = v[2 * j + 1];
      rope_pair(ci.rf_hi[j], ci.rf_lo[j], p, lo[j], hi[j]);
    }
  };
  switch (ci.seg) {
    case 0: {
      T *dst = reinterpret_cast<T *>(e.q) + (size_t)row * Wa;
      if constexpr (ROPE == ROPE_PAIRED_COLS) {
        float lo[W / 2], hi[W / 2];
        turn(lo, hi);
        const int base = ci.c - ci.c % e.hd, i0 = (ci.c % e.hd) >> 1;
        storeW_T<T, W / 2>(dst + base + i0, lo);
        storeW_T<T, W / 2>(dst + base + e.hd / 2 + i0, hi);
        return;
      }
      storeW_T<T, W>(dst + ci.c, v);
      return;
    }
    case 1:
    case 2: {
      const bool isv = ci.seg == 2;
      const int G = e.KV / e.hd;
      // dims d0.. of the head get the W values (n at most W), for every copy
      auto put = [&](int d0, const float *vals, auto width) {
        constexpr int WW = decltype(width)::value;
        if (e.mode == EPI_DECODE) {
          const int p = e.len[row];
          if (p < 0 || (!e.is_ring && p >= e.cap)) return;
          const int slot = e.is_ring ? p % e.cap : p;
          T *dst = reinterpret_cast<T *>(isv ? e.cache_v : e.cache_k);
          storeW_T<T, WW>(dst + (((size_t)row * G + ci.g) * e.cap + slot) * e.hd + d0, vals);
          return;
        }
        const int n = e.n_rows_per_seq;
        const int b = row / n, p = row - b * n;
        T *full = reinterpret_cast<T *>(isv ? e.v_full : e.k_full);
        storeW_T<T, WW>(full + (((size_t)b * G + ci.g) * n + p) * e.hd + d0, vals);
        if (e.mode == EPI_PREFILL && e.cache_k) {
          const bool keep = e.is_ring ? (p >= n - e.cap) : (p < e.cap);
          if (keep) {
            const int slot = e.is_ring ? p % e.cap : p;
            T *dst = reinterpret_cast<T *>(isv ? e.cache_v : e.cache_k);
            storeW_T<T, WW>(dst + (((size_t)b * G + ci.g) * e.cap + slot) * e.hd + d0, vals);
          }
        }
      };
      if (ROPE == ROPE_PAIRED_COLS && !isv) {
        float lo[W / 2], hi[W / 2];
        turn(lo, hi);
        const int i0 = ci.d >> 1;
        put(i0, lo, std::integral_constant<int, W / 2>{});
        put(e.hd / 2 + i0, hi, std::integral_constant<int, W / 2>{});
        return;
      }
      put(ci.d, v, std::integral_constant<int, W>{});
      return;
    }
    // a group of W columns (W divides 64, col % W == 0) never crosses a
    // 64-column block, so it stays one vector store in either layout
    case 3: storeW_T<float, W>(e.xs + ssm_at(e, row, ci.c, D), v); return;
    case 4: storeW_T<T, W>(reinterpret_cast<T *>(e.z) + ssm_at(e, row, ci.c, D), v); return;
    case 5: {
      float sp[W];
#pragma unroll
      for (int i = 0; i < W; ++i) sp[i] = softplus_f(v[i] + ci.bias[i]);
      storeW_T<float, W>(e.dt + ssm_at(e, row, ci.c, e.Ddt), sp);
      return;
    }
    default: storeW_T<float, W>(e.bc + (size_t)row * 2 * e.N + ci.c, v); return;
  }
}

// ROPE_SPLIT_GROUPS: a lane's two groups of one row, dims d..d+W-1 (ci0, va)
// and d+hd/2.. (ci1, vb) of the same Q or K head, turned pairwise and stored;
// other blocks of the map are stored as they are.
template <class T, int W, int ROPE>
__device__ __forceinline__ void inproj_store_pair(const InProjOut &e, int row, const ColInfo<W> &ci0,
                                                  const float va[W], const ColInfo<W> &ci1,
                                                  const float vb[W]) {
  if (ROPE == ROPE_SPLIT_GROUPS && (ci0.seg == 0 || ci0.seg == 1)) {
    const float p = (float)rope_position(e, row);
    float x[W], y[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      x[j] = va[j];
      y[j] = vb[j];
      rope_pair(ci0.rf_hi[j], ci0.rf_lo[j], p, x[j], y[j]);
    }
    inproj_storeW<T, W, ROPE_NONE>(e, row, ci0, x);
    inproj_storeW<T, W, ROPE_NONE>(e, row, ci1, y);
    return;
  }
  inproj_storeW<T, W, ROPE>(e, row, ci0, va);
  inproj_storeW<T, W, ROPE>(e, row, ci1, vb);
}

// ---- launchers (each returns hipGetLastError() of its launches) ------------
// `part`: split-K scratch of skinny_part_bytes(M, K, Ncols) bytes (bf16 path
// with few rows); may be null when that size is 0.
template <class T>
hipError_t launch_inproj(const T *x, int M, int K, const T *w, int Ncols,
                         const InProjOut &epi, float *part, hipStream_t s);
// out = f w^T (+ resid when it is not null: the block's residual add)
template <class T>
hipError_t launch_outproj(const T *f, int M, int K, const T *w, int Ncols, T *out,
                          const T *resid, float *part, hipStream_t s);
// The block MLP's first projection: w holds gate and up rows alternately
// (Ncols = 2 d_ff); h[M, d_ff] = SiLU(gate) * up
template <class T>
hipError_t launch_mlp_gate_up(const T *x, int M, int K, const T *w, int Ncols, T *h,
                              float *part, hipStream_t s);
// The fusion of Eq. (3) folded into the output projection (bf16, many rows):
// the attention and SSM branches store beta-scaled outputs and per-row sums of
// squares of the unscaled ones (ssq_o: G partials per row, one per KV group;
// ssq_y: one per 64-channel block), and
//   out[r] = s_o(r) (beta_a O)[r] W_a^T + s_y(r) (beta_y Y)[r] W_y^T,
//   s(r) = 1 / (2 sqrt(mean of squares + eps)),
// W = [W_a | W_y] the output-projection rows split at column Wa.  The GEMM
// walks the Y columns first, rescales its accumulators by s_y / s_o, walks
// the O columns and multiplies by s_o before the epilogue.
struct NormScale {
  const void *y;           // [M, D] beta_y Y (the A operand's columns Wa..Wa+D)
  const float *ssq_o;      // [M, go]
  const float *ssq_y;      // [M, gy]
  int Wa, D, go, gy;
  float eps;
};
// out = [o | y] w^T with the row scales of ns (+ resid); o is [M, Wa]
template <class T>
hipError_t launch_outproj_fused(const T *o, const NormScale &ns, int M, const T *w, int Ncols, T *out,
                                const T *resid, hipStream_t s);
// whether launch_outproj_fused takes this shape (bf16, many rows, Wa and D
// whole k-tiles)
bool outproj_fused_ok(int M, int Wa, int D);
size_t skinny_part_bytes(int M, int K, int N);
// compute units of the current device (256 if the query fails)
int device_cus();

struct AttnArgs {
  const void *q;           // [B*n, H*hd]
  const void *k, *v;       // real keys [B, G, n, hd]
  const void *mk, *mv;     // meta keys [G, m, hd]
  void *o;                 // [B*n, H*hd]
  int B, n, m, H, G, hd, window, is_global;
  // fused norm (bf16): o holds beta * O and ssq[row * G + g] the sum of the
  // group's unscaled O^2 over its heads' columns; null: plain O
  const float *beta;       // [H*hd]
  float *ssq;              // [B*n, G]
  // the producer's cache now holds the prompt: set_len[0..set_len_n) =
  // set_len_value (written by the first workgroup); null: nothing
  int32_t *set_len;
  int set_len_n, set_len_value;
};
template <class T> hipError_t launch_attention(const AttnArgs &a, hipStream_t s);

struct ScanArgs {
  // xs, z and dt in the channel-block-major layout over B*n rows (ssm_index)
  const float *xs;         // [B*n, D] fp32
  const void *z;           // [B*n, D] (null: no gate, no Y)
  const float *dt;         // [B*n, D], or [B*n, S] for Mamba2 heads
  const float *bc;         // [B*n, 2N]
  const float *A;          // [D, N], or [S] for Mamba2 heads
  const float *conv_w;     // [D, k]
  const float *conv_b;     // [D]
  const float *h0;         // [D, N] initial state (null: zero)
  const float *tail0;      // [k-1, D] fp32 conv history (null: zero)
  void *y;                 // [B*n, D] (null: not written)
  float *h_out;            // [B, D, N] (null: not written)
  float *tail_out;         // [B, k-1, D] fp32 (null: not written)
  float *carry;            // workspace for chunk carries
  int B, n, D, N, k;
  int chunk;               // time steps per chunk
  int S;                   // Mamba2 heads (per-head Delta, scalar A); 0: Mamba
  int ck0, b0;             // pass 1: chunk and sequence of the grid's first workgroup
  // fused norm: y holds beta * Y and ssq[row * ceil(D/64) + c/64] the sum of
  // unscaled Y^2 over the 64-channel block; null: plain Y
  const float *beta;       // [D]
  float *ssq;              // [B*n, ceil(D/64)]
};
template <class T> hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
// The scan in two parts, for a caller that overlaps the first with other
// work: launch_scan_summaries runs pass 1 over chunks [ck0, ck1) of sequences
// [b0, b1) (the chunk summaries; chunks from nc - 1 on have none);
// launch_scan_finish runs pass 2 and pass 3 once every summary is written.
template <class T>
hipError_t launch_scan_summaries(const ScanArgs &a, int ck0, int ck1, int b0, int b1, hipStream_t s);
template <class T> hipError_t launch_scan_finish(const ScanArgs &a, hipStream_t s);
// pass 2 alone (the carries), for a caller that runs pass 3 in the launch
// beside the attention (launch_attn_scan3)
template <class T> hipError_t launch_scan_carries(const ScanArgs &a, hipStream_t s);
// The attention (aa) and scan pass 3 (sa) in one grid whose workgroups take
// either role (bf16 only; pass 1 and pass 2 of sa must have run)
template <class T> hipError_t launch_attn_scan3(const AttnArgs &aa, const ScanArgs &sa, hipStream_t s);
int scan_chunks(const ScanArgs &a);
size_t scan_carry_bytes(int B, int n, int D, int N, int *chunk_out);

struct NormArgs {
  const void *o;           // [rows, Wa]
  const void *y;           // [rows, D]
  const float *beta_attn, *beta_ssm;
  void *f;                 // [rows, Wa + D]
  int rows, Wa, D;
  float eps;
  // decode: when part is set the attention half is merged from the split
  // partials of the decode attention (o unused); Wa = H * hd
  const float *part;
  int H, hd, nsplit;
  // prefill of a producer with a cache: set_len[0..set_len_n) = set_len_value
  // (the cache now holds the prompt's positions); null: nothing
  int32_t *set_len;
  int set_len_n, set_len_value;
  // decode step of a producer: its new token joins the cache, len[b] += 1 for
  // b < bump_n (a ring always, a linear cache while below bump_cap); the norm
  // runs after every reader of len in the step (attention); null: nothing
  int32_t *len_bump;
  int bump_n, bump_cap, bump_ring;
};
template <class T> hipError_t launch_norm_fuse(const NormArgs &a, hipStream_t s);
// out[r] = g * x[r] / sqrt(mean(x[r]^2) + eps) for each of `rows` rows of d
// values (the block's pre-norms); d a multiple of 8 (bf16) or 4 (fp32)
template <class T>
hipError_t launch_rmsnorm(const T *x, const float *g, T *out, int rows, int d, float eps,
                          hipStream_t s);

struct DecodeAttnArgs {
  const void *q;           // [B, H*hd]
  const void *cache_k, *cache_v;  // [B, G, cap, hd]
  const void *mk, *mv;     // [G, m, hd]
  const int32_t *len;
  int producer;            // 1: new token at len[b]; 0: at len[b]-1
  void *o;                 // [B, H*hd]
  float *part;             // split partials
  int B, H, G, hd, m, cap, is_ring, window, is_global, split, nsplit;
};
// Per-split partials sit at part[((b*H + h)*nsplit + s)*(hd + 2)]: the running
// maximum m of the base-2 scaled scores, l = sum 2^(score - m), then
// a[hd] = sum 2^(score - m) v.  The merge of several splits is left to the
// caller (the decode norm does it); *o_ready says whether o holds the
// finished output (one split, written directly).
template <class T>
hipError_t launch_decode_attention(const DecodeAttnArgs &a, hipStream_t s, bool *o_ready);
size_t decode_attn_part_bytes(int B, int H, int G, int hd, int m, int max_real,
                              int *split_out, int *nsplit_out);

struct DecodeSsmArgs {
  const float *xs;         // [B, D] fp32
  const void *z;           // [B, D]
  const float *dt, *bc;    // [B, D] (Mamba2: [B, S]), [B, 2N]
  const float *A, *conv_w, *conv_b;   // A [D, N] (Mamba2: [S])
  float *h;                // [B, D, N] in/out
  float *conv;             // [B, k-1, D] fp32 in/out
  void *y;                 // [B, D]
  int B, D, N, k;
  int S;                   // Mamba2 heads; 0: Mamba
};
template <class T> hipError_t launch_decode_ssm(const DecodeSsmArgs &a, hipStream_t s);


}  // namespace hh

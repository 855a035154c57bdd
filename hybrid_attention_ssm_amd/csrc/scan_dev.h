// Device code of the SSM heads' prefill scan, shared by the scan kernels
// and the launch that runs scan pass 3 beside the attention (the method is
// described in scan.hip).  Everything here is per wavefront: one wave owns
// 64 channels of one chunk, its LDS buffers are its own, and it synchronises
// only with itself, so a workgroup may hold several independent scan waves.
#pragma once
#include "hh_internal.h"

namespace hh {
namespace sdev {

// LDS written by this wave is visible to its later reads (the wave's LDS
// operations complete in order; the fences keep the compiler from moving
// accesses across)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int NS = 16;      // SSM state size
constexpr int KC = 4;       // conv taps held (shorter kernels are zero-padded)
constexpr int TB = 8;       // time steps loaded per batch

struct ChanParams {
  float A2[NS];             // A * log2(e) (Mamba2: A2[0] is the head's)
  float w[KC];              // conv taps, w[KC-1] multiplies the current row
  float bias;
  float beta;               // fused norm: the channel's beta (else 1)
  int dcol;                 // Delta of this channel: its column
};

template <bool SC>
__device__ __forceinline__ void load_params(const ScanArgs &a, int c, ChanParams &p) {
  if constexpr (SC) {
    const int h = c / (a.D / a.S);
    p.A2[0] = a.A[h] * kLog2e;
    p.dcol = h;
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) p.A2[s] = a.A[(size_t)c * NS + s] * kLog2e;
    p.dcol = c;
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int src = j - (KC - a.k);          // zero-pad taps in front
    p.w[j] = src >= 0 ? a.conv_w[(size_t)c * a.k + src] : 0.0f;
  }
  p.bias = a.conv_b[c];
  p.beta = a.beta ? a.beta[c] : 1.0f;
}

// history: hist[0] = xs_{t0-1}, hist[1] = xs_{t0-2}, hist[2] = xs_{t0-3}
template <class T>
__device__ __forceinline__ void load_history(const ScanArgs &a, int b, int c, int t0, float hist[KC - 1]) {
  const float *xs = a.xs;
  const float *tail = a.tail0;
  const size_t R = (size_t)a.B * a.n;
#pragma unroll
  for (int j = 0; j < KC - 1; ++j) {
    const int pos = t0 - 1 - j;
    float v = 0.0f;
    if (pos >= 0) v = xs[ssm_index((size_t)b * a.n + pos, c, R)];
    else if (tail && (a.k - 1) + pos >= 0) v = tail[(size_t)((a.k - 1) + pos) * a.D + c];
    hist[j] = v;
  }
}

// One time step of the channel recurrence.  bc points at B_t then C_t (the
// same for every channel, so the loads are uniform).
template <int MODE, bool SC>
__device__ __forceinline__ float scan_step(const ChanParams &p, float h[NS], float hist[KC - 1],
                                           float x, float dt, const float bv[NS],
                                           const float cv[NS], float &dsum) {
  const float conv = p.bias + p.w[3] * x + p.w[2] * hist[0] + p.w[1] * hist[1] + p.w[0] * hist[2];
  hist[2] = hist[1];
  hist[1] = hist[0];
  hist[0] = x;
  const float du = dt * silu_f(conv);
  float acc = 0.0f;
  const float decay1 = SC ? exp2_fast(dt * p.A2[0]) : 0.0f;   // Mamba2: one per step
  if constexpr (!SC) {
    // all decays first: 16 independent exponentials for the scheduler to
    // interleave, instead of 16 dependent mul -> exp -> FMA chains
    float dec[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) dec[s] = exp2_fast(dt * p.A2[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      h[s] = fmaf(dec[s], h[s], du * bv[s]);
      if (MODE == 1 || MODE == 2) acc = fmaf(cv[s], h[s], acc);
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float decay = SC ? decay1 : exp2_fast(dt * p.A2[s]);
      h[s] = fmaf(decay, h[s], du * bv[s]);
      if (MODE == 1 || MODE == 2) acc = fmaf(cv[s], h[s], acc);
    }
  }
  if (MODE == 0) dsum += dt;
  return acc;
}

// The scan over [t0, t1) of sequence b for channel c.  MODE 0: summary
// (end state and sum of Delta); MODE 1: Y; MODE 2: Y and its row sums of
// squares (fused norm); MODE 3: no Y (only the final state and history).
// B_t/C_t are the same for every channel: SUB steps of them are staged in LDS
// (sbc, SUB*2N floats) and read back as broadcasts; per-lane inputs are read
// TB steps at a time.
constexpr int SUB = 64;

// Fused norm (sq not null): each output step's unscaled Y^2 goes to row
// (step % TB) of sq (TB x 65 floats, one column per lane).  After each batch
// of TB steps (and after the block's last steps) lane l adds the 8 columns
// 8(l%8).. of row l/8 and three DPP steps combine the 8 lanes of a row,
// giving the row's sum over the wave's 64 channels.
constexpr int SQ_LD = 65;
static_assert(TB == 8, "one sq row per lane group of 8");

template <class T, int MODE, bool SC>
__device__ __forceinline__ void scan_range(const ScanArgs &a, int b, int c, bool active, int t0,
                                           int t1, const ChanParams &p, float h[NS],
                                           float hist[KC - 1], float &dsum, float *sbc,
                                           float *sq, int cb, int ncb) {
  constexpr bool HAS_Y = MODE == 1 || MODE == 2;
  const T *z = reinterpret_cast<const T *>(a.z);
  const size_t D = a.D;
  const size_t row0 = (size_t)b * a.n;
  const size_t R = (size_t)a.B * a.n;
  // this lane's column of xs, Delta and z from the sequence's first row:
  // step t is element t * 64 (channel-block-major layout)
  const float *xs = a.xs + ssm_index(row0, c, R);
  const float *dtp = a.dt + ssm_index(row0, p.dcol, R);
  const T *zp = HAS_Y ? z + ssm_index(row0, c, R) : nullptr;
  const int lane = threadIdx.x & 63;
  // Y is stored through a buffer resource based at the block's first row, so
  // a step's address is a scalar offset; lanes past the last channel get an
  // offset past the buffer's end, which the hardware drops
  const unsigned yoff = active ? (unsigned)c * sizeof(T) : 0x80000000u;
  for (int s0 = t0; s0 < t1; s0 += SUB) {
    const int len = min(SUB, t1 - s0);
    // (MODE 0 / 3: a.y may be null; the resource is then never used)
    const __amdgpu_buffer_rsrc_t rsY = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<T *>(a.y) + (HAS_Y ? (row0 + s0) * D : 0), (short)0,
        HAS_Y ? (int)(len * D * sizeof(T)) : 0, 0x00020000);
    // Y of block step tt (the output: beta * Y; its square to sq row tt % TB)
    auto emit = [&](int tt, float yv) {
      const int so = tt * (int)(D * sizeof(T));
      if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<T>(p.beta * yv)),
                                              rsY, yoff, so, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, from_f32<T>(p.beta * yv)),
                                              rsY, yoff, so, 0);
      if constexpr (MODE == 2) sq[(tt % TB) * SQ_LD + lane] = active ? yv * yv : 0.0f;
    };
    // the row sums of block steps base .. base + rows - 1
    auto flush = [&](int base, int rows) {
      __builtin_amdgcn_wave_barrier();
      const int r = lane >> 3, q = lane & 7;
      float acc2 = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc2 += sq[r * SQ_LD + q * 8 + j];
      // xor 1 and xor 2 inside each quad (quad_perm), then the mirrored lane
      // of the same 8 (row_half_mirror: l <-> 7 - l, the other quad)
      acc2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc2), 0xB1, 0xF, 0xF, false));
      acc2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc2), 0x4E, 0xF, 0xF, false));
      acc2 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc2), 0x141, 0xF, 0xF, false));
      if (q == 0 && r < rows) a.ssq[(row0 + s0 + base + r) * ncb + cb] = acc2;
      __builtin_amdgcn_wave_barrier();
    };
    wave_sync();   // previous block's reads are done
    // all loads first, then the LDS writes (indices past the block repeat
    // its last vector, so every load is unconditional)
    const float4 *src = reinterpret_cast<const float4 *>(a.bc + (row0 + s0) * (2 * NS));
    constexpr int PER_LANE = SUB * (2 * NS / 4) / 64;
    const int last = len * (2 * NS / 4) - 1;
    float4 stage[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) stage[j] = src[min(lane + 64 * j, last)];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) reinterpret_cast<float4 *>(sbc)[min(lane + 64 * j, last)] = stage[j];
    wave_sync();
    int t = 0;
    // per-lane inputs of batch t are loaded one batch ahead (the loads of
    // batch t+TB are in flight while batch t is computed); the prefetch past
    // the last full batch re-reads that batch (a cache hit)
    float xv[TB], dv[TB];
    T zv[TB];
    // (one base address per batch; the steps' offsets are immediates)
    auto load_batch = [&](int tb, float (&xo)[TB], float (&dvo)[TB], T (&zo)[TB]) {
      const size_t base = (size_t)(s0 + tb) * 64;
      const float *xb = xs + base, *db = dtp + base;
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        xo[i] = xb[i * 64];
        dvo[i] = db[i * 64];
      }
      if constexpr (HAS_Y) {
        const T *zb = zp + base;
#pragma unroll
        for (int i = 0; i < TB; ++i) zo[i] = zb[i * 64];
      }
    };
    if (TB <= len) load_batch(0, xv, dv, zv);
    for (; t + TB <= len; t += TB) {
      float xn[TB], dn[TB];
      T zn[TB];
      load_batch(t + 2 * TB <= len ? t + TB : t, xn, dn, zn);
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        const float4 *bc4 = reinterpret_cast<const float4 *>(sbc + (t + i) * 2 * NS);
        float bv[NS], cv[NS];
#pragma unroll
        for (int q = 0; q < NS / 4; ++q) {
          const float4 v = bc4[q];
          bv[4 * q] = v.x; bv[4 * q + 1] = v.y; bv[4 * q + 2] = v.z; bv[4 * q + 3] = v.w;
          if (HAS_Y) {
            const float4 u = bc4[NS / 4 + q];
            cv[4 * q] = u.x; cv[4 * q + 1] = u.y; cv[4 * q + 2] = u.z; cv[4 * q + 3] = u.w;
          }
        }
        const float acc = scan_step<MODE, SC>(p, h, hist, xv[i], dv[i], bv, cv, dsum);
        if constexpr (HAS_Y) emit(t + i, acc * silu_f(to_f32(zv[i])));
      }
      if constexpr (MODE == 2) flush(t, TB);
#pragma unroll
      for (int i = 0; i < TB; ++i) { xv[i] = xn[i]; dv[i] = dn[i]; zv[i] = zn[i]; }
    }
    const int t_rest = t;
    for (; t < len; ++t) {
      const size_t idx = (size_t)(s0 + t) * 64;
      const float4 *bc4 = reinterpret_cast<const float4 *>(sbc + t * 2 * NS);
      float bv[NS], cv[NS];
#pragma unroll
      for (int q = 0; q < NS / 4; ++q) {
        const float4 v = bc4[q];
        bv[4 * q] = v.x; bv[4 * q + 1] = v.y; bv[4 * q + 2] = v.z; bv[4 * q + 3] = v.w;
        if (HAS_Y) {
          const float4 u = bc4[NS / 4 + q];
          cv[4 * q] = u.x; cv[4 * q + 1] = u.y; cv[4 * q + 2] = u.z; cv[4 * q + 3] = u.w;
        }
      }
      const float acc = scan_step<MODE, SC>(p, h, hist, xs[idx], dtp[idx], bv, cv, dsum);
      if constexpr (HAS_Y) emit(t, acc * silu_f(to_f32(zp[idx])));
    }
    if constexpr (MODE == 2) if (t_rest < len) flush(t_rest, len - t_rest);
  }
}


// Scan pass 3 for one wave: chunk ck of sequence b, channel block cb (64
// channels), from the chunk's true entry state (h0 for the first chunk, the
// carry of pass 2 otherwise); writes Y (OUT 1, 2), the row sums (OUT 2) and,
// in the last chunk, the final state and conv history.  sbc: SUB * 2N floats
// of LDS; sq: TB * SQ_LD floats (OUT 2).
template <class T, bool SC, int OUT>
__device__ __forceinline__ void pass3_wave(const ScanArgs &a, int ck, int cb, int b, float *sbc, float *sq) {
  const int lane = threadIdx.x & 63;
  const int ncb = (a.D + 63) / 64;
  // lanes past the last channel compute a copy of it (every lane takes part
  // in staging B/C) and store nothing
  const bool active = cb * 64 + lane < a.D;
  const int c = min(cb * 64 + lane, a.D - 1);
  const int nc = (a.n + a.chunk - 1) / a.chunk;
  ChanParams p;
  load_params<SC>(a, c, p);
  const int t0 = ck * a.chunk, t1 = min(a.n, t0 + a.chunk);
  float hist[KC - 1];
  load_history<T>(a, b, c, t0, hist);
  float h[NS];
  if (ck == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) h[s] = a.h0 ? a.h0[(size_t)c * NS + s] : 0.0f;
  } else {
    const float *hs = a.carry + ((size_t)b * nc + ck - 1) * NS * a.D;
#pragma unroll
    for (int s = 0; s < NS; ++s) h[s] = hs[(size_t)s * a.D + c];
  }
  float dsum = 0.0f;
  scan_range<T, OUT, SC>(a, b, c, active, t0, t1, p, h, hist, dsum, sbc, sq, cb, ncb);
  if (ck == nc - 1 && active) {
    if (a.h_out) {
      float *ho = a.h_out + ((size_t)b * a.D + c) * NS;
#pragma unroll
      for (int s = 0; s < NS; s += 4)
        *reinterpret_cast<float4 *>(ho + s) = make_float4(h[s], h[s + 1], h[s + 2], h[s + 3]);
    }
    if (a.tail_out) {
      float *to = a.tail_out + (size_t)b * (a.k - 1) * a.D;
      for (int j = 0; j < a.k - 1; ++j) to[(size_t)j * a.D + c] = hist[a.k - 2 - j];
    }
  }
}

// the pass-3 output mode of a call: 1 Y, 2 Y and row sums, 3 no Y
__host__ __device__ inline int pass3_mode(const ScanArgs &a) { return !a.y ? 3 : a.ssq ? 2 : 1; }

}  // namespace sdev
}  // namespace hh

// SSM heads of the hybrid-head layer, prefill
// (Hymba paper §2.1 Eq. (2): the Mamba selective scan with input-dependent
// Delta, B, C and the output gate G; the conv1d + SiLU on the SSM input and
// SiLU on the gate follow Mamba, which the paper adopts for its SSM heads).
//
//   u_t = SiLU(conv_b + sum_j conv_w[j] * xs_{t-(k-1)+j})
//   h_t = exp(Delta_t A) * h_{t-1} + Delta_t u_t B_t      (per channel, N states)
//   y_t = h_t . C_t,   Y_t = y_t * SiLU(z_t)
//
// One lane owns one channel and keeps its N = 16 states in registers; B_t and
// C_t are the same for every channel, so each wavefront reads them as uniform
// (scalar) loads while xs, Delta and z are read coalesced across 64 channels.
// exp(Delta A) is evaluated as 2^(Delta * A log2 e).
//
// Time is cut into chunks so that a single sequence fills the GPU:
//   pass 1 (chunks 0..C-2): scan each chunk from a zero state; keep its end
//          state and sum(Delta) (the chunk's total decay is exp(A sum Delta));
//   pass 2: per channel, combine the chunk summaries in order starting from
//          the meta state h0: H_c = exp(A S_c) H_{c-1} + h_c;
//   pass 3 (all chunks): rescan each chunk from its true incoming state and
//          write Y; the last chunk writes the final state and conv history.
// With one chunk only pass 3 runs.
//
// Mamba2 heads (a.S > 0, template flag SC): the P = D / S channels of a head
// share Delta_t and one scalar A, so the decay exp(Delta A) is one exp2 per
// (step, channel) for all N states instead of N.
#include "hh_internal.h"

namespace hh {

namespace {
constexpr int NS = 16;      // SSM state size
constexpr int KC = 4;       // conv taps held (shorter kernels are zero-padded)
constexpr int TB = 8;       // time steps loaded per batch

struct ChanParams {
  float A2[NS];             // A * log2(e) (Mamba2: A2[0] is the head's)
  float w[KC];              // conv taps, w[KC-1] multiplies the current row
  float bias;
  int dcol, dstride;        // Delta of this channel: column and row stride
};

template <bool SC>
__device__ __forceinline__ void load_params(const ScanArgs &a, int c, ChanParams &p) {
  if constexpr (SC) {
    const int h = c / (a.D / a.S);
    p.A2[0] = a.A[h] * kLog2e;
    p.dcol = h;
    p.dstride = a.S;
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) p.A2[s] = a.A[(size_t)c * NS + s] * kLog2e;
    p.dcol = c;
    p.dstride = a.D;
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int src = j - (KC - a.k);          // zero-pad taps in front
    p.w[j] = src >= 0 ? a.conv_w[(size_t)c * a.k + src] : 0.0f;
  }
  p.bias = a.conv_b[c];
}

// history: hist[0] = xs_{t0-1}, hist[1] = xs_{t0-2}, hist[2] = xs_{t0-3}
template <class T>
__device__ __forceinline__ void load_history(const ScanArgs &a, int b, int c, int t0, float hist[KC - 1]) {
  const float *xs = a.xs;
  const float *tail = a.tail0;
#pragma unroll
  for (int j = 0; j < KC - 1; ++j) {
    const int pos = t0 - 1 - j;
    float v = 0.0f;
    if (pos >= 0) v = xs[((size_t)b * a.n + pos) * a.D + c];
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
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float decay = SC ? decay1 : exp2_fast(dt * p.A2[s]);
    h[s] = fmaf(decay, h[s], du * bv[s]);
    if (MODE == 1) acc = fmaf(cv[s], h[s], acc);
  }
  if (MODE == 0) dsum += dt;
  return acc;
}

// The scan over [t0, t1) of sequence b for channel c.  MODE 0: summary
// (end state and sum of Delta); MODE 1: output (Y, and final state/history).
// B_t/C_t are the same for every channel: SUB steps of them are staged in LDS
// (sbc, SUB*2N floats) and read back as broadcasts; per-lane inputs are read
// TB steps at a time.
constexpr int SUB = 64;

template <class T, int MODE, bool SC>
__device__ __forceinline__ void scan_range(const ScanArgs &a, int b, int c, bool active, int t0,
                                           int t1, const ChanParams &p, float h[NS],
                                           float hist[KC - 1], float &dsum, float *sbc) {
  const float *xs = a.xs;
  const T *z = reinterpret_cast<const T *>(a.z);
  T *y = reinterpret_cast<T *>(a.y);
  // without Y the gate is not needed: read (and ignore) xs instead, so the
  // loads stay unconditional
  const T *zp = y ? z : reinterpret_cast<const T *>(xs);
  const size_t D = a.D;
  const size_t row0 = (size_t)b * a.n;
  const int lane = threadIdx.x;
  for (int s0 = t0; s0 < t1; s0 += SUB) {
    const int len = min(SUB, t1 - s0);
    __syncthreads();   // previous block's reads are done
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
    __syncthreads();
    int t = 0;
    // per-lane inputs of batch t are loaded one batch ahead (the loads of
    // batch t+TB are in flight while batch t is computed); the prefetch past
    // the last full batch re-reads that batch (a cache hit)
    float xv[TB], dv[TB];
    T zv[TB];
    auto load_batch = [&](int tb, float (&xo)[TB], float (&dvo)[TB], T (&zo)[TB]) {
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        const size_t idx = (row0 + s0 + tb + i) * D + c;
        xo[i] = xs[idx];
        dvo[i] = a.dt[(row0 + s0 + tb + i) * p.dstride + p.dcol];
        if (MODE == 1) zo[i] = zp[idx];
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
          if (MODE == 1) {
            const float4 u = bc4[NS / 4 + q];
            cv[4 * q] = u.x; cv[4 * q + 1] = u.y; cv[4 * q + 2] = u.z; cv[4 * q + 3] = u.w;
          }
        }
        const float acc = scan_step<MODE, SC>(p, h, hist, xv[i], dv[i], bv, cv, dsum);
        if (MODE == 1 && y && active)
          y[(row0 + s0 + t + i) * D + c] = from_f32<T>(acc * silu_f(to_f32(zv[i])));
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) { xv[i] = xn[i]; dv[i] = dn[i]; zv[i] = zn[i]; }
    }
    for (; t < len; ++t) {
      const size_t idx = (row0 + s0 + t) * D + c;
      const float4 *bc4 = reinterpret_cast<const float4 *>(sbc + t * 2 * NS);
      float bv[NS], cv[NS];
#pragma unroll
      for (int q = 0; q < NS / 4; ++q) {
        const float4 v = bc4[q];
        bv[4 * q] = v.x; bv[4 * q + 1] = v.y; bv[4 * q + 2] = v.z; bv[4 * q + 3] = v.w;
        if (MODE == 1) {
          const float4 u = bc4[NS / 4 + q];
          cv[4 * q] = u.x; cv[4 * q + 1] = u.y; cv[4 * q + 2] = u.z; cv[4 * q + 3] = u.w;
        }
      }
      const float acc = scan_step<MODE, SC>(p, h, hist, xs[idx],
                                            a.dt[(row0 + s0 + t) * p.dstride + p.dcol], bv, cv, dsum);
      if (MODE == 1 && y && active) y[idx] = from_f32<T>(acc * silu_f(to_f32(z[idx])));
    }
  }
}

}  // namespace

// pass 1: summaries of chunks 0..C-2.  grid (C-1, ceil(D/64), B), 64 threads
template <class T, bool SC>
__global__ void __launch_bounds__(64) scan_pass1(ScanArgs a) {
  const int ck = blockIdx.x, b = blockIdx.z;
  // lanes past the last channel compute a copy of it (every lane takes part
  // in staging B/C) and store nothing
  const bool active = blockIdx.y * 64 + (int)threadIdx.x < a.D;
  const int c = min(blockIdx.y * 64 + (int)threadIdx.x, a.D - 1);
  const int nc = (a.n + a.chunk - 1) / a.chunk;
  ChanParams p;
  load_params<SC>(a, c, p);
  const int t0 = ck * a.chunk, t1 = min(a.n, t0 + a.chunk);
  float hist[KC - 1];
  load_history<T>(a, b, c, t0, hist);
  float h[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) h[s] = 0.0f;
  float dsum = 0.0f;
  __shared__ float4 sbc[SUB * 2 * NS / 4];
  scan_range<T, 0, SC>(a, b, c, active, t0, t1, p, h, hist, dsum, reinterpret_cast<float *>(sbc));
  // carry layout: [B][nc][NS][D] states, then [B][nc][D] delta sums
  if (!active) return;
  float *hs = a.carry + ((size_t)b * nc + ck) * NS * a.D;
#pragma unroll
  for (int s = 0; s < NS; ++s) hs[(size_t)s * a.D + c] = h[s];
  float *ds = a.carry + (size_t)a.B * nc * NS * a.D;
  ds[((size_t)b * nc + ck) * a.D + c] = dsum;
}

// pass 2: chunk carries in order.  One lane per (channel, state) recurrence;
// the loads of a group of chunks do not depend on the carry, so they are
// issued together.  grid (ceil(N*D/256), B), 256 threads
__global__ void __launch_bounds__(256) scan_pass2(ScanArgs a) {
  constexpr int U = 8;
  const int b = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= NS * a.D) return;
  const int s = idx / a.D, c = idx - s * a.D;
  const int nc = (a.n + a.chunk - 1) / a.chunk;
  const float A2 = (a.S ? a.A[c / (a.D / a.S)] : a.A[(size_t)c * NS + s]) * kLog2e;
  float H = a.h0 ? a.h0[(size_t)c * NS + s] : 0.0f;
  const float *ds = a.carry + (size_t)a.B * nc * NS * a.D + (size_t)b * nc * a.D + c;
  float *hs = a.carry + ((size_t)b * nc * NS + s) * a.D + c;
  const size_t hstride = (size_t)NS * a.D;
  for (int c0 = 0; c0 + 1 < nc; c0 += U) {
    float Sv[U], hv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ck = c0 + u;
      const bool in = ck + 1 < nc;
      Sv[u] = in ? ds[(size_t)ck * a.D] : 0.0f;
      hv[u] = in ? hs[ck * hstride] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ck = c0 + u;
      if (ck + 1 >= nc) break;
      H = fmaf(exp2_fast(A2 * Sv[u]), H, hv[u]);
      hs[ck * hstride] = H;               // state entering chunk ck+1
    }
  }
}

// pass 3: outputs of every chunk.  grid (C, ceil(D/64), B)
template <class T, bool SC>
__global__ void __launch_bounds__(64) scan_pass3(ScanArgs a) {
  const int ck = blockIdx.x, b = blockIdx.z;
  // lanes past the last channel compute a copy of it (every lane takes part
  // in staging B/C) and store nothing
  const bool active = blockIdx.y * 64 + (int)threadIdx.x < a.D;
  const int c = min(blockIdx.y * 64 + (int)threadIdx.x, a.D - 1);
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
  __shared__ float4 sbc[SUB * 2 * NS / 4];
  scan_range<T, 1, SC>(a, b, c, active, t0, t1, p, h, hist, dsum, reinterpret_cast<float *>(sbc));
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

size_t scan_carry_bytes(int B, int n, int D, int N, int *chunk_out) {
  // enough (channel-wave x chunk) work items to fill 256 CUs several times
  const int cw = (D + 63) / 64;
  const long waves = (long)B * cw;
  int nc = (int)((4096 + waves - 1) / waves);
  nc = std::max(1, std::min(nc, (n + 63) / 64));
  int chunk = (n + nc - 1) / nc;
  chunk = (chunk + 7) / 8 * 8;
  if (chunk < 8) chunk = 8;
  nc = (n + chunk - 1) / chunk;
  if (chunk_out) *chunk_out = chunk;
  return (size_t)B * nc * (N + 1) * D * sizeof(float);
}

template <class T, bool SC>
static hipError_t launch_scan_t(const ScanArgs &a, hipStream_t s) {
  const int nc = (a.n + a.chunk - 1) / a.chunk;
  const int cw = (a.D + 63) / 64;
  if (nc > 1) {
    hipLaunchKernelGGL((scan_pass1<T, SC>), dim3(nc - 1, cw, a.B), dim3(64), 0, s, a);
    hipLaunchKernelGGL(scan_pass2, dim3((NS * a.D + 255) / 256, a.B), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((scan_pass3<T, SC>), dim3(nc, cw, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
  return a.S ? launch_scan_t<T, true>(a, s) : launch_scan_t<T, false>(a, s);
}

template hipError_t launch_scan<float>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan<bf16>(const ScanArgs &, hipStream_t);

}  // namespace hh

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
// C_t are the same for every channel, so each wavefront reads them as
// broadcasts from LDS, while xs, Delta and z arrive in the channel-block-major
// layout (ssm_index): a wave's 64 channels are one contiguous 256-byte run per
// time step, and consecutive steps are adjacent runs, so each wave streams its
// chunk as one contiguous region.
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
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float decay = SC ? decay1 : exp2_fast(dt * p.A2[s]);
    h[s] = fmaf(decay, h[s], du * bv[s]);
    if (MODE == 1 || MODE == 2) acc = fmaf(cv[s], h[s], acc);
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
                                           float *sq = nullptr) {
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
  const int lane = threadIdx.x;
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
      if (q == 0 && r < rows) a.ssq[(row0 + s0 + base + r) * gridDim.y + blockIdx.y] = acc2;
      __builtin_amdgcn_wave_barrier();
    };
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

}  // namespace

// pass 1: summaries of chunks 0..C-2.  grid (C-1, ceil(D/64), B), 64 threads
template <class T, bool SC>
__global__ void __launch_bounds__(64) scan_pass1(ScanArgs a) {
  const int ck = a.ck0 + (int)blockIdx.x, b = a.b0 + (int)blockIdx.z;
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

// pass 2: chunk carries.  Per (channel, state) the chunk summaries compose
// as affine maps, H_k = exp(A S_k) H_{k-1} + h_k (S_k the chunk's sum of
// Delta, h_k its end state from zero).  A group of G2 lanes shares one
// (channel, state): lane j owns a run of consecutive chunks, loads all their
// summaries at once and composes them from zero into one map; the G2 maps are
// scanned across the group with lane shuffles (log2 G2 steps), which gives
// each lane its run's entry state; the lane then walks its run again and
// writes the state entering every following chunk.  grid (ceil(N*D*G2/256),
// B), 256 threads.
constexpr int P2_RUN = 24;   // chunks per lane at most

template <int G2>
__global__ void __launch_bounds__(256) scan_pass2(ScanArgs a) {
  const int b = blockIdx.y;
  const int gid = (blockIdx.x * 256 + (int)threadIdx.x) / G2;   // (state, channel) index
  const int j = (int)threadIdx.x % G2;                           // lane in the group
  const bool live = gid < NS * a.D;
  const int idx = live ? gid : 0;
  const int s = idx / a.D, c = idx - s * a.D;
  const int nc = (a.n + a.chunk - 1) / a.chunk;
  const int ncar = nc - 1;                       // carries to produce
  const int run = (ncar + G2 - 1) / G2;          // <= P2_RUN (checked by the launcher)
  const int k0 = min(j * run, ncar), k1 = min(k0 + run, ncar);
  const float A2 = (a.S ? a.A[c / (a.D / a.S)] : a.A[(size_t)c * NS + s]) * kLog2e;
  const float *ds = a.carry + (size_t)a.B * nc * NS * a.D + (size_t)b * nc * a.D + c;
  float *hs = a.carry + ((size_t)b * nc * NS + s) * a.D + c;
  const size_t hstride = (size_t)NS * a.D;
  float Sv[P2_RUN], hv[P2_RUN];
#pragma unroll
  for (int u = 0; u < P2_RUN; ++u) {
    const bool in = live && k0 + u < k1;
    Sv[u] = in ? ds[(size_t)(k0 + u) * a.D] : 0.0f;
    hv[u] = in ? hs[(k0 + u) * hstride] : 0.0f;
  }
  // this lane's run as one map H -> P H + g
  float P = 1.0f, g = 0.0f;
#pragma unroll
  for (int u = 0; u < P2_RUN; ++u) {
    if (k0 + u >= k1) break;
    const float d = exp2_fast(A2 * Sv[u]);
    P *= d;
    g = fmaf(d, g, hv[u]);
  }
  // inclusive scan of the maps over the group (lane j composes lanes 0..j,
  // the earlier map applied first), then shift to exclusive
#pragma unroll
  for (int off = 1; off < G2; off <<= 1) {
    const float Pp = __shfl_up(P, off, G2), gp = __shfl_up(g, off, G2);
    if (j >= off) {
      g = fmaf(P, gp, g);
      P *= Pp;
    }
  }
  float Pe = __shfl_up(P, 1, G2), ge = __shfl_up(g, 1, G2);
  if (j == 0) { Pe = 1.0f; ge = 0.0f; }
  const float h0 = a.h0 ? a.h0[(size_t)c * NS + s] : 0.0f;
  float H = fmaf(Pe, h0, ge);                     // state entering chunk k0
  if (!live) return;
#pragma unroll
  for (int u = 0; u < P2_RUN; ++u) {
    if (k0 + u >= k1) break;
    H = fmaf(exp2_fast(A2 * Sv[u]), H, hv[u]);
    hs[(k0 + u) * hstride] = H;                 // state entering chunk k0+u+1
  }
}

// pass 3: outputs of every chunk.  grid (C, ceil(D/64), B).  OUT: the
// scan_range mode (1: Y, 2: Y and row sums of squares, 3: no Y)
template <class T, bool SC, int OUT>
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
  __shared__ float sq[OUT == 2 ? TB * SQ_LD : 1];
  scan_range<T, OUT, SC>(a, b, c, active, t0, t1, p, h, hist, dsum, reinterpret_cast<float *>(sbc), sq);
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
  // at most 64 * P2_RUN + 1 chunks, so pass 2's lane groups hold every carry
  nc = std::max(1, std::min({nc, (n + 63) / 64, 1024}));
  int chunk = (n + nc - 1) / nc;
  chunk = (chunk + 7) / 8 * 8;
  if (chunk < 8) chunk = 8;
  nc = (n + chunk - 1) / chunk;
  if (chunk_out) *chunk_out = chunk;
  return (size_t)B * nc * (N + 1) * D * sizeof(float);
}

int scan_chunks(const ScanArgs &a) { return (a.n + a.chunk - 1) / a.chunk; }

template <class T, bool SC>
static hipError_t launch_summaries_t(const ScanArgs &a0, int ck0, int ck1, int b0, int b1, hipStream_t s) {
  const int nc = scan_chunks(a0);
  ck1 = std::min(ck1, nc - 1);
  if (ck0 >= ck1 || b0 >= b1) return hipSuccess;
  ScanArgs a = a0;
  a.ck0 = ck0;
  a.b0 = b0;
  const int cw = (a.D + 63) / 64;
  hipLaunchKernelGGL((scan_pass1<T, SC>), dim3(ck1 - ck0, cw, b1 - b0), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <class T, bool SC>
static hipError_t launch_finish_t(const ScanArgs &a, hipStream_t s) {
  const int nc = scan_chunks(a);
  const int cw = (a.D + 63) / 64;
  if (nc > 1) {
    // lanes per (channel, state) group: the fewest whose runs hold every carry
    const int ncar = nc - 1;
    const int g2 = ncar <= 4 * P2_RUN ? 4 : ncar <= 16 * P2_RUN ? 16 : ncar <= 64 * P2_RUN ? 64 : 0;
    if (!g2) return hipErrorInvalidValue;
    const dim3 grid2((unsigned)(((long)NS * a.D * g2 + 255) / 256), a.B);
    if (g2 == 4) hipLaunchKernelGGL(scan_pass2<4>, grid2, dim3(256), 0, s, a);
    else if (g2 == 16) hipLaunchKernelGGL(scan_pass2<16>, grid2, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(scan_pass2<64>, grid2, dim3(256), 0, s, a);
  }
  const dim3 grid3(nc, cw, a.B);
  if (!a.y) hipLaunchKernelGGL((scan_pass3<T, SC, 3>), grid3, dim3(64), 0, s, a);
  else if (a.ssq) hipLaunchKernelGGL((scan_pass3<T, SC, 2>), grid3, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((scan_pass3<T, SC, 1>), grid3, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_scan_summaries(const ScanArgs &a, int ck0, int ck1, int b0, int b1, hipStream_t s) {
  return a.S ? launch_summaries_t<T, true>(a, ck0, ck1, b0, b1, s)
             : launch_summaries_t<T, false>(a, ck0, ck1, b0, b1, s);
}

template <class T>
hipError_t launch_scan_finish(const ScanArgs &a, hipStream_t s) {
  return a.S ? launch_finish_t<T, true>(a, s) : launch_finish_t<T, false>(a, s);
}

template <class T>
hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
  hipError_t e = launch_scan_summaries<T>(a, 0, scan_chunks(a), 0, a.B, s);
  return e == hipSuccess ? launch_scan_finish<T>(a, s) : e;
}

template hipError_t launch_scan_summaries<float>(const ScanArgs &, int, int, int, int, hipStream_t);
template hipError_t launch_scan_summaries<bf16>(const ScanArgs &, int, int, int, int, hipStream_t);
template hipError_t launch_scan_finish<float>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan_finish<bf16>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan<float>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan<bf16>(const ScanArgs &, hipStream_t);

}  // namespace hh

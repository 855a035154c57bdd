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
#include "scan_dev.h"

namespace hh {

using namespace sdev;

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
  scan_range<T, 0, SC>(a, b, c, active, t0, t1, p, h, hist, dsum, reinterpret_cast<float *>(sbc), nullptr,
                       blockIdx.y, gridDim.y);
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

// pass 3: outputs of every chunk.  grid (C, ceil(D/64), B), one wave per
// workgroup.  OUT: the scan_range mode (1: Y, 2: Y and row sums of squares,
// 3: no Y)
template <class T, bool SC, int OUT>
__global__ void __launch_bounds__(64) scan_pass3(ScanArgs a) {
  __shared__ float4 sbc[SUB * 2 * NS / 4];
  __shared__ float sq[OUT == 2 ? TB * SQ_LD : 1];
  pass3_wave<T, SC, OUT>(a, blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<float *>(sbc), sq);
}

size_t scan_carry_bytes(int B, int n, int D, int N, int *chunk_out) {
  // Passes 1 and 3 run one wave per (chunk, 64 channels, sequence).  At three
  // waves per SIMD (their register budget) 256 CUs hold kScanSlots of them at
  // once, and a wave that finds no slot waits for a whole wave's time.  The
  // chunk is the shortest multiple of 8 steps (at least 64; at most 1024
  // chunks, so pass 2's lane groups hold every carry) whose waves all fit in
  // one round, or whose full chunks do while the last is at most a quarter
  // as long: its waves finish early and hand their slots to the few that did
  // not fit.  8k, one sequence: 62 chunks of 136 steps (the last 24),
  // against 80 chunks of 104 steps (1.3 rounds): scan 192-195 against
  // 199-201 us on one box.
  constexpr long kScanSlots = 3 * 4 * 256;
  const long wpc = (long)B * ((D + 63) / 64);   // waves per chunk index
  int chunk = std::max(64, ((n + 1023) / 1024 + 7) / 8 * 8);
  for (; chunk < n; chunk += 8) {
    const long full = n / chunk, rem = n % chunk;
    if ((full + (rem ? 1 : 0)) * wpc <= kScanSlots ||
        (full * wpc <= kScanSlots && 4L * rem <= chunk))
      break;
  }
  chunk = std::min(chunk, std::max(n, 1));
  const int nc = (n + chunk - 1) / chunk;
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
static hipError_t launch_finish_t(const ScanArgs &a, hipStream_t s, bool pass3 = true) {
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
  if (!pass3) return hipGetLastError();
  const dim3 grid3(nc, cw, a.B);
  const int mode = pass3_mode(a);
  if (mode == 3) hipLaunchKernelGGL((scan_pass3<T, SC, 3>), grid3, dim3(64), 0, s, a);
  else if (mode == 2) hipLaunchKernelGGL((scan_pass3<T, SC, 2>), grid3, dim3(64), 0, s, a);
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
hipError_t launch_scan_carries(const ScanArgs &a, hipStream_t s) {
  return a.S ? launch_finish_t<T, true>(a, s, false) : launch_finish_t<T, false>(a, s, false);
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
template hipError_t launch_scan_carries<float>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan_carries<bf16>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan<float>(const ScanArgs &, hipStream_t);
template hipError_t launch_scan<bf16>(const ScanArgs &, hipStream_t);

}  // namespace hh

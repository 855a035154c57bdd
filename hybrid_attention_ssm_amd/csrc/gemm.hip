// Input and output projections of the hybrid-head layer
// (Hymba paper, §2.1: the fused W_in_proj of the design formulation, and
// Eq. (3)'s W_out_proj).
//
// C[M, N] = A[M, K] B[N, K]^T with A, B row-major and K contiguous ("NT"), so
// both operands are read along K.  bf16 path: MFMA v_mfma_f32_32x32x16_bf16
// with fp32 accumulators; the fp32 path uses a plain LDS-tiled FMA kernel.
// Results go through an epilogue functor (the in-projection splits its
// columns into Q, K/V (+ cache slots), xs, z, softplus(dt + b), B, C).
#include "hh_internal.h"

namespace hh {

// Map the linear block id to an output tile.  Hardware hands consecutive
// block ids to the 8 XCDs in turn; the remap gives each XCD a contiguous run
// of logical tiles, and the grouped order (GROUP row-tiles per column sweep)
// keeps the A rows and B columns of that run in the XCD's own L2.  Logical
// column tiles alternate between the left and right halves of the output, so
// each XCD's run mixes both: column blocks whose epilogue costs more (the
// in-projection's softplus columns sit at its right end) are spread over all
// XCDs instead of piling onto half of them.
__device__ __forceinline__ bool tile_of(int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int GROUP = 8;
  int bid = blockIdx.x;
  const int nb = gridDim.x;  // a multiple of 8
  bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (bid >= tiles_m * tiles_n) return false;
  const int group_size = GROUP * tiles_n;
  const int first_m = (bid / group_size) * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int in_group = bid % group_size;
  tm = first_m + in_group % gm;
  const int lt = in_group / gm;
  tn = (lt & 1) ? (tiles_n + 1) / 2 + (lt >> 1) : (lt >> 1);
  return true;
}

// An epilogue may remap which row of B (the weights) feeds output column n
// (src_row; the in-projection does for RoPE).  Without one, row n.
template <class E, class = void> struct HasRowMap : std::false_type {};
template <class E>
struct HasRowMap<E, std::void_t<decltype(&E::src_row)>> : std::true_type {};
template <class Epi>
__device__ __forceinline__ int b_row(const Epi &epi, int n) {
  if constexpr (HasRowMap<Epi>::value) return epi.src_row(n);
  else return n;
}
// An epilogue may also take a lane's two column groups of a row together
// (store_pair; the in-projection's rotary embedding pairs them).
template <class E, class = void> struct HasPairStore : std::false_type {};
template <class E>
struct HasPairStore<E, std::void_t<decltype(&E::template store_pair<4>)>> : std::true_type {};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, operands streamed straight into LDS
//
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes at the instruction's
// LDS base + 16*l, so each lane fetches the global chunk that belongs at its
// (swizzled) LDS slot.  k-tiles are 32 wide and STAGES deep: the loads of
// tile kt+STAGES-1 are issued while tile kt is multiplied, giving the global
// reads STAGES-1 tiles of MFMA time to land.  Waits and barriers are explicit
// (s_waitcnt vmcnt + s_barrier) so nothing drains the load pipeline.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int BK_ = 32>
struct LdsCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int BK = BK_;                     // bf16 per k-tile row (32 or 64)
  static constexpr int KCH = BK / 8;                 // 16-byte chunks per row
  static constexpr int KS = BK / 16;                 // MFMA k-steps per k-tile
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_UNITS = BM * KCH, B_UNITS = BN * KCH;   // 16-byte units
  static constexpr int STAGE = A_UNITS + B_UNITS;
  // a stage is A_Q + B_Q load instructions of 64 x 16 bytes, dealt round the
  // waves; when they do not divide evenly, the last waves repeat the first
  // instructions (the same bytes into the same slots), so every wave issues
  // the same count and waits for the same vmcnt
  static constexpr int A_Q = A_UNITS / 64, B_Q = B_UNITS / 64;
  static constexpr int A_INS = (A_Q + NWAVES - 1) / NWAVES;   // load instrs per wave
  static constexpr int B_INS = (B_Q + NWAVES - 1) / NWAVES;
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(A_Q * 64 == A_UNITS && B_Q * 64 == B_UNITS, "tile rows");
  // chunk c of row `row` sits at slot c ^ f(row): the 16 (32) rows one
  // fragment read touches with the same c land on distinct 16-byte bank groups
  __device__ static __forceinline__ int swz(int row, int c) {
    return BK == 32 ? row * 4 + (c ^ ((row >> 2) & 3)) : row * 8 + (c ^ ((row >> 1) & 7));
  }
};

// FUSED (the output projection under the fused norm, see NormScale): A is
// [M, ns.Wa] with K = ns.Wa + ns.D, its columns continued by ns.y [M, ns.D];
// the k-tiles of the y part run first, then the accumulators are rescaled by
// s_y / s_o, then the o part, then the accumulators are multiplied by s_o.
// Rows of a lane's A fragments are lr (A layout); accumulator element r of
// a 32x32 block belongs to row 8(r/4) + 4lh + r%4 (C layout).
template <class Cfg, class Epi, bool FUSED = false>
__global__ void __launch_bounds__(Cfg::NT)
gemm_bf16_lds(const bf16 *__restrict__ A, const bf16 *__restrict__ B, int M, int N, int K, Epi epi,
              NormScale ns) {
  // the body uses LDS-DMA builtins that exist only for the device target; the
  // host pass needs just the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ uint4 smem[Cfg::STAGES * Cfg::STAGE];
  int tm, tn;
  if (!tile_of((M + Cfg::BM - 1) / Cfg::BM, (N + Cfg::BN - 1) / Cfg::BN, tm, tn)) return;
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int lr = lane & 31, lh = lane >> 5;

  // buffers based at the tile's first row; rows past M (N) read as zero
  const int lda = FUSED ? ns.Wa : K;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(A + (size_t)m0 * lda), (short)0, (M - m0) * lda * 2, 0x00020000);
  __amdgpu_buffer_rsrc_t rsY = rsA;
  if constexpr (FUSED)
    rsY = __builtin_amdgcn_make_buffer_rsrc((void *)(static_cast<const bf16 *>(ns.y) + (size_t)m0 * ns.D),
                                            (short)0, (M - m0) * ns.D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(B + (size_t)n0 * K), (short)0, (N - n0) * K * 2, 0x00020000);
  int voffA[Cfg::A_INS], voffB[Cfg::B_INS], voffY[FUSED ? Cfg::A_INS : 1];
  auto qA = [&](int j) { return (wave * Cfg::A_INS + j) % Cfg::A_Q; };   // instruction of the stage
  auto qB = [&](int j) { return (wave * Cfg::B_INS + j) % Cfg::B_Q; };
#pragma unroll
  for (int j = 0; j < Cfg::A_INS; ++j) {   // LDS unit u holds chunk of swz(row, kc) == u
    const int u = qA(j) * 64 + lane;
    const int row = u / Cfg::KCH, kc = Cfg::swz(row, u % Cfg::KCH) - row * Cfg::KCH;
    voffA[j] = (row * lda + kc * 8) * 2;
    if constexpr (FUSED) voffY[j] = (row * ns.D + kc * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < Cfg::B_INS; ++j) {
    const int u = qB(j) * 64 + lane;
    const int row = u / Cfg::KCH, kc = Cfg::swz(row, u % Cfg::KCH) - row * Cfg::KCH;
    voffB[j] = ((b_row(epi, n0 + row) - n0) * K + kc * 8) * 2;
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto issue = [&](int kt, int st) {
    const int soff = kt * Cfg::BK * 2;
    uint4 *base = smem + st * Cfg::STAGE;
    if (FUSED && kt * Cfg::BK >= ns.Wa) {   // a k-tile of the y part
#pragma unroll
      for (int j = 0; j < Cfg::A_INS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsY, (lds_void *)(base + qA(j) * 64), 16, voffY[FUSED ? j : 0], soff - ns.Wa * 2, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < Cfg::A_INS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsA, (lds_void *)(base + qA(j) * 64), 16, voffA[j], soff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < Cfg::B_INS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void *)(base + Cfg::A_UNITS + qB(j) * 64), 16, voffB[j],
          soff, 0, 0);
  };

  f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragments of k-step ks (16 deep) sit in buffer ks % 2
  bf16x8 af[2][Cfg::TM], bfr[2][Cfg::TN];
  auto fload = [&](const uint4 *sA, int ks) {
    const uint4 *sB = sA + Cfg::A_UNITS;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
      af[ks & 1][i] = __builtin_bit_cast(bf16x8, sA[Cfg::swz(wm * Cfg::WM + i * 32 + lr, ks * 2 + lh)]);
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
      bfr[ks & 1][j] = __builtin_bit_cast(bf16x8, sB[Cfg::swz(wn * Cfg::WN + j * 32 + lr, ks * 2 + lh)]);
  };
  auto mfmas = [&](int ks) {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
  };

  // split-K: slice blockIdx.y of gridDim.y covers k-tiles [kt0, kt0 + ktiles)
  const int ktiles_all = K / Cfg::BK;
  const int kps = (ktiles_all + gridDim.y - 1) / gridDim.y;
  const int kt0 = blockIdx.y * kps;
  const int ktiles = max(0, min(ktiles_all - kt0, kps));
  // steps past the end repeat the last; FUSED starts at the y part's first k-tile
  const int n_y = FUSED ? ns.D / Cfg::BK : 0, n_o = FUSED ? ns.Wa / Cfg::BK : 0;
  auto ktile = [&](int i) {
    const int t = min(i, ktiles - 1);
    return FUSED ? (t < n_y ? n_o + t : t - n_y) : kt0 + t;
  };
  // FUSED: each lane's row scales s_o, s_y (A layout), from the partial sums
  // of squares: lane half lh = 0 adds the o partials and the first half of
  // the y partials, lh = 1 the rest
  float rso[Cfg::TM], rsy[Cfg::TM];
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int row = m0 + wm * Cfg::WM + i * 32 + lr;
      float po = 0.0f, py = 0.0f;
      // PCH loads in flight at a time, then their sum
      constexpr int PCH = 16;
      auto add_run = [&](const float *p, int cnt, float &acc) {
        for (int g0 = 0; g0 < cnt; g0 += PCH) {
          float v[PCH];
#pragma unroll
          for (int j = 0; j < PCH; ++j) v[j] = g0 + j < cnt ? p[g0 + j] : 0.0f;
#pragma unroll
          for (int j = 0; j < PCH; ++j) acc += v[j];
        }
      };
      if (row < M) {
        if (lh == 0) add_run(ns.ssq_o + (size_t)row * ns.go, ns.go, po);
        const int half = ns.gy / 2;
        const int y0 = lh == 0 ? 0 : half, y1 = lh == 0 ? half : ns.gy;
        add_run(ns.ssq_y + (size_t)row * ns.gy + y0, y1 - y0, py);
      }
      const float qo = __shfl_xor(po, 32), qy = __shfl_xor(py, 32);
      po = lh == 0 ? po + qo : qo + po;   // the same order in both halves
      py = lh == 0 ? py + qy : qy + py;
      rso[i] = 0.5f / sqrtf(po / (float)ns.Wa + ns.eps);
      rsy[i] = 0.5f / sqrtf(py / (float)ns.D + ns.eps);
    }
  }
  // multiply accumulator rows by v (given in the A layout)
  auto scale_rows = [&](const float (&v)[Cfg::TM]) {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float f = __shfl(v[i], 8 * (r >> 2) + 4 * lh + (r & 3));
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) acc[i][j][r] *= f;
      }
  };
  auto stage = [&](int kt) { return smem + (kt % Cfg::STAGES) * Cfg::STAGE; };
  // in a scheduling region holding one k-step's MFMAs and the next k-step's
  // fragment reads, alternate the two (an MFMA first: it needs no new read)
  // so the reads are in flight under the MFMAs instead of queued behind all
  // of them
  auto interleave = [&]() {
    constexpr int NR = Cfg::TM + Cfg::TN, NM = Cfg::TM * Cfg::TN;
    constexpr int P = NR < NM ? NR : NM;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    if constexpr (NM > P) __builtin_amdgcn_sched_group_barrier(0x008, NM - P, 0);
    if constexpr (NR > P) __builtin_amdgcn_sched_group_barrier(0x100, NR - P, 0);
  };
  constexpr int PER_TILE = Cfg::A_INS + Cfg::B_INS;
  // Software pipeline per k-tile kt (its stage holds tile kt): each k-step's
  // fragments are read while the previous k-step's MFMAs run; after the
  // first k-step the stage of tile kt-1 is refilled with tile kt+STAGES-1
  // (every wave passed the barrier after its last read of it); before the
  // last k-step's MFMAs (their fragments are already in registers) wait for
  // tile kt+1, barrier, and read its first fragments under those MFMAs.
#pragma unroll
  for (int st = 0; st < Cfg::STAGES - 1; ++st) issue(ktile(st), st);
  wait_vmcnt<(Cfg::STAGES - 2) * PER_TILE>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  fload(stage(0), 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    const uint4 *sA = stage(kt);
    if constexpr (FUSED) {
      if (kt == n_y) {   // the y part is done: acc = s_y/s_o * (beta_y Y) W_y^T
        float ratio[Cfg::TM];
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i) ratio[i] = rsy[i] / rso[i];
        scale_rows(ratio);
      }
    }
#pragma unroll
    for (int ks = 0; ks + 1 < Cfg::KS; ++ks) {
      fload(sA, ks + 1);
      mfmas(ks);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      if (ks == 0) {
        const int nt = kt + Cfg::STAGES - 1;
        issue(ktile(nt), nt % Cfg::STAGES);
      }
    }
    // the last k-step's fragments are in registers: sync first, then read the
    // next tile's first fragments under its MFMAs
    wait_vmcnt<(Cfg::STAGES - 2) * PER_TILE>();   // this wave's loads of tile kt+1 have landed
    wait_lgkmcnt0();                             // its reads of tile kt are done
    __builtin_amdgcn_s_barrier();               // ... and every other wave's
    __builtin_amdgcn_sched_barrier(0);
    fload(stage(kt + 1), 0);                     // (past the last tile: a harmless re-read)
    mfmas(Cfg::KS - 1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  if constexpr (FUSED) scale_rows(rso);

  // the wave's WN columns are staged CW at a time (all of them when WN <= 64)
  constexpr int CW = Cfg::WN % 64 == 0 ? 64 : 32;
  static_assert(Cfg::WN % CW == 0 && (CW == Cfg::WN || CW == 32), "epilogue chunks");
  constexpr int SROW = CW + 8;
  constexpr int LPR = CW / 8;   // lanes per row; each stores two groups of 4 columns
  constexpr int RPI = 64 / LPR;
  static_assert(Cfg::NWAVES * 32 * SROW * 4 <= (int)sizeof(smem), "epilogue strip fits");
  float *strip = reinterpret_cast<float *>(smem) + wave * 32 * SROW;
  // a lane stores columns c0..c0+3 and CW/2+c0..+3 of every row it visits, so
  // each store instruction writes one contiguous run per row; the routing of
  // both groups is resolved once per chunk
  const int c0 = (lane % LPR) * 4, c1 = CW / 2 + c0;
#pragma unroll
  for (int ch = 0; ch < Cfg::WN / CW; ++ch) {
    const int g0 = n0 + wn * Cfg::WN + ch * CW + c0, g1 = n0 + wn * Cfg::WN + ch * CW + c1;
    const bool ok0 = g0 < N, ok1 = g1 < N;
    const typename Epi::template Col<4> ci0 = epi.template col_info<4>(ok0 ? g0 : 0);
    const typename Epi::template Col<4> ci1 = epi.template col_info<4>(ok1 ? g1 : 0);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
      for (int jj = 0; jj < CW / 32; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          strip[(8 * (r >> 2) + 4 * lh + (r & 3)) * SROW + jj * 32 + lr] = acc[i][ch * (CW / 32) + jj][r];
      // the strip is this wave's own: LDS keeps one wave's accesses in order,
      // so only the compiler must not move the reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // with 64 LDS banks a float4 read serves 16 lanes per cycle: when they
      // are two rows of 8 lanes (CW = 64), take rows r and r + 4 (4 SROW
      // floats apart, 128 bytes mod 256) rather than r and r + 1
      const int q = lane / LPR;
      const int qrow = (LPR == 8 && RPI == 8) ? ((q & 1) << 2) | (q >> 1) : q;
#pragma unroll 1
      for (int it = 0; it < 32 / RPI; ++it) {
        const int rr = it * RPI + qrow;
        const float4 a = *reinterpret_cast<const float4 *>(strip + rr * SROW + c0);
        const float4 b = *reinterpret_cast<const float4 *>(strip + rr * SROW + c1);
        const float va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {b.x, b.y, b.z, b.w};
        const int row = m0 + wm * Cfg::WM + i * 32 + rr;
        if (row < M) {
          if constexpr (HasPairStore<Epi>::value) {
            if (ok0 && ok1) {
              epi.template store_pair<4>(row, ci0, va, ci1, vb);
              continue;
            }
          }
          if (ok0) epi.template store<4>(row, ci0, va);
          if (ok1) epi.template store<4>(row, ci1, vb);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64x64 tile, k-step 16, 4x4 outputs per thread
// ---------------------------------------------------------------------------
template <class Epi>
__global__ void __launch_bounds__(256)
gemm_f32_tiled(const float *__restrict__ A, const float *__restrict__ B, int M, int N, int K,
               Epi epi) {
  __shared__ float sA[16][64 + 4];
  __shared__ float sB[16][64 + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + i * 256;
      const int r = e >> 4, kk = e & 15;
      sA[kk][r] = (m0 + r < M && k0 + kk < K) ? A[(size_t)(m0 + r) * K + k0 + kk] : 0.0f;
      sB[kk][r] = (n0 + r < N && k0 + kk < K) ? B[(size_t)b_row(epi, n0 + r) * K + k0 + kk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  // each thread's 4 columns form one epilogue group (N % 4 == 0)
  const int col = n0 + tx * 4;
  if (col >= N) return;
  const typename Epi::template Col<4> ci = epi.template col_info<4>(col);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row < M) epi.template store<4>(row, ci, acc[i]);
  }
}

// ---------------------------------------------------------------------------
// epilogues and launchers
// ---------------------------------------------------------------------------
// Epilogue interface: col_info<W>(col) resolves, once per lane, a group of W
// consecutive output columns (col % W == 0); store<W>(row, info, v) writes
// the group's W values of one row.
// ROPE (a RopeMode): how Q and K meet the rotary embedding in the epilogue;
// under ROPE_PAIRED_COLS the weight rows of their heads are read in pair
// order (src_row), under ROPE_SPLIT_GROUPS the kernel's lane owns both
// halves of its pairs (store_pair)
template <class T, int ROPE>
struct InProjEpi {
  InProjOut e;
  template <int W> using Col = ColInfo<W>;
  __device__ __forceinline__ int src_row(int n) const {
    return ROPE == ROPE_PAIRED_COLS ? inproj_src_row(e, n) : n;
  }
  template <int W>
  __device__ __forceinline__ Col<W> col_info(int col) const { return inproj_col<W, ROPE>(e, col); }
  template <int W>
  __device__ __forceinline__ void store(int row, const Col<W> &ci, const float v[W]) const {
    inproj_storeW<T, W, ROPE>(e, e.row0 + row, ci, v);
  }
  template <int W>
  __device__ __forceinline__ void store_pair(int row, const Col<W> &ci0, const float va[W],
                                             const Col<W> &ci1, const float vb[W]) const {
    inproj_store_pair<T, W, ROPE>(e, e.row0 + row, ci0, va, ci1, vb);
  }
};

template <class T>
struct StoreEpi {
  T *out;
  int ld;
  template <int W> using Col = int;
  template <int W>
  __device__ __forceinline__ int col_info(int col) const { return col; }
  template <int W>
  __device__ __forceinline__ void store(int row, int col, const float v[W]) const {
    storeW_T<T, W>(out + (size_t)row * ld + col, v);
  }
};

// out = sum + resid, both [M, ld] (the block's residual add)
template <class T>
struct ResidEpi {
  T *out;
  const T *resid;
  int ld;
  template <int W> using Col = int;
  template <int W>
  __device__ __forceinline__ int col_info(int col) const { return col; }
  template <int W>
  __device__ __forceinline__ void store(int row, int col, const float v[W]) const {
    float r[W];
    loadW_T<T, W>(resid + (size_t)row * ld + col, r);
#pragma unroll
    for (int i = 0; i < W; ++i) r[i] += v[i];
    storeW_T<T, W>(out + (size_t)row * ld + col, r);
  }
};

// Columns arrive as (gate, up) pairs (the block MLP's interleaved rows):
// h[row, col/2 + i] = SiLU(gate_i) * up_i, W/2 outputs per group.
template <class T>
struct GluEpi {
  T *h;
  int ld;   // d_ff
  template <int W> using Col = int;
  template <int W>
  __device__ __forceinline__ int col_info(int col) const { return col; }
  template <int W>
  __device__ __forceinline__ void store(int row, int col, const float v[W]) const {
    float o[W / 2];
#pragma unroll
    for (int i = 0; i < W / 2; ++i) o[i] = silu_f(v[2 * i]) * v[2 * i + 1];
    storeW_T<T, W / 2>(h + (size_t)row * ld + col / 2, o);
  }
};

// Split-K partial sums: slice blockIdx.y of the K range writes fp32 to its
// own [M, N] plane.
struct PartialEpi {
  float *part;
  int M, N;
  template <int W> using Col = int;
  template <int W>
  __device__ __forceinline__ int col_info(int col) const { return col; }
  template <int W>
  __device__ __forceinline__ void store(int row, int col, const float v[W]) const {
    storeW_T<float, W>(part + ((size_t)blockIdx.y * M + row) * N + col, v);
  }
};

// Sum the split-K planes and hand each 4-column group to the real epilogue.
// Every split's load is issued before the first add (splits <= kMaxSplits).
constexpr int kMaxSplits = 16;
template <class Epi>
__global__ void __launch_bounds__(256)
reduce_splits(const float *__restrict__ part, int splits, int M, int N, Epi epi) {
  const int groups = N / 4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)M * groups) return;
  const int row = (int)(idx / groups), col = (int)(idx % groups) * 4;
  float4 p[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < splits) p[sp] = *reinterpret_cast<const float4 *>(part + ((size_t)sp * M + row) * N + col);
  float v[4] = {0, 0, 0, 0};
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < splits) { v[0] += p[sp].x; v[1] += p[sp].y; v[2] += p[sp].z; v[3] += p[sp].w; }
  epi.template store<4>(row, epi.template col_info<4>(col), v);
}

template <class Cfg, class Epi>
static hipError_t run_lds(const bf16 *A, int M, int K, const bf16 *B, int N, const Epi &epi,
                          hipStream_t s) {
  const int tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
  const int grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_bf16_lds<Cfg, Epi>), dim3(grid), dim3(Cfg::NT), 0, s, A, B, M, N, K,
                     epi, NormScale{});
  return hipGetLastError();
}

// 256x256 tile, 8 waves of 128x64 (two per SIMD, so one wave's LDS waits and
// barriers hide behind the other's MFMAs), 3 LDS stages (96 KB)
using CfgLds = LdsCfg<256, 256, 128, 64, 3>;
// 256x224 tile, 8 waves of 32x224: for outputs whose 256x256 tiles leave part
// of the chip idle in their last round (8192 x 1600: 224 tiles on 256 CUs,
// with 12% padding), 224-wide tiles give every CU one tile of 7/8 the area.
// 64-deep k-tiles in 2 stages (120 KB): half the barriers of 32-deep ones,
// whose per-k-tile sync costs this shape more (its waves read the whole
// 224-row B tile); needs K (and, fused, both parts of K) a multiple of 64
using CfgWide = LdsCfg<256, 224, 32, 224, 2, 64>;
// Few rows (decode, meta prefix): the weights dominate the traffic and each
// workgroup streams a slab of 64 weight rows.  When those slabs alone leave
// the chip short of workgroups (the output projection: 25 slabs) the K range
// is split too; fp32 partials are then summed by reduce_splits, which applies
// the epilogue.  `part` holds splits*M*N floats.  (A split input projection
// loses more to its partial planes and the scattered epilogue of the reduce
// than it gains.)  Each workgroup re-reads all M rows of the activations from
// L2, which bounds it; 64-deep k-tiles halve its barriers and double the bytes
// per DMA batch, and 8 waves of 32x32 keep more loads in flight.
using CfgSkinny = LdsCfg<128, 64, 32, 32, 4, 64>;
constexpr int kSkinnyTargetWG = 200;   // workgroups a few-row GEMM aims for

static int skinny_splits(int M, int K, int N) {
  using C = CfgSkinny;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  if (tiles >= 128) return 1;
  const int ktiles = K / C::BK;
  const int splits = std::max(1, std::min({ktiles / 8, (kSkinnyTargetWG + tiles - 1) / tiles, kMaxSplits}));
  const int kps = (ktiles + splits - 1) / splits;
  return (ktiles + kps - 1) / kps;   // no empty slice
}

template <class Cfg, class Epi>
static hipError_t run_skinny_cfg(const bf16 *A, int M, int K, const bf16 *B, int N, const Epi &epi,
                                 int splits, float *part, hipStream_t s) {
  const int tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
  const int grid = (tiles + 7) / 8 * 8;
  if (splits == 1) {
    hipLaunchKernelGGL((gemm_bf16_lds<Cfg, Epi>), dim3(grid), dim3(Cfg::NT), 0, s, A, B, M, N, K,
                       epi, NormScale{});
    return hipGetLastError();
  }
  PartialEpi pe{part, M, N};
  hipLaunchKernelGGL((gemm_bf16_lds<Cfg, PartialEpi>), dim3(grid, splits), dim3(Cfg::NT), 0, s, A,
                     B, M, N, K, pe, NormScale{});
  const long groups = (long)M * (N / 4);
  hipLaunchKernelGGL((reduce_splits<Epi>), dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s,
                     part, splits, M, N, epi);
  return hipGetLastError();
}

template <class Epi>
static hipError_t run_skinny(const bf16 *A, int M, int K, const bf16 *B, int N, const Epi &epi,
                             float *part, hipStream_t s) {
  return run_skinny_cfg<CfgSkinny>(A, M, K, B, N, epi, part ? skinny_splits(M, K, N) : 1, part, s);
}

// rounds of one-tile-per-CU times the tile's area: the many-row kernel's time
// up to its per-flop efficiency
template <class Cfg>
static long tile_cost(int M, int N, int cus) {
  const long tiles = (long)((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
  return (tiles + cus - 1) / cus * (long)Cfg::BM * Cfg::BN;
}

// the wide tile reads more LDS per flop: only where it saves a tenth (and
// where its deeper k-tiles divide K)
static bool use_wide(int M, int N, int K) {
  const int cus = device_cus();
  return K % CfgWide::BK == 0 && 10 * tile_cost<CfgWide>(M, N, cus) < 9 * tile_cost<CfgLds>(M, N, cus);
}

template <class Epi>
static hipError_t run_bf16_auto(const bf16 *A, int M, int K, const bf16 *B, int N, const Epi &epi,
                                float *part, hipStream_t s) {
  if (M >= 1024) {
    if (use_wide(M, N, K)) return run_lds<CfgWide>(A, M, K, B, N, epi, s);
    return run_lds<CfgLds>(A, M, K, B, N, epi, s);
  }
  return run_skinny(A, M, K, B, N, epi, part, s);
}

template <class Cfg, class Epi>
static hipError_t run_fused(const bf16 *o, const NormScale &ns, int M, const bf16 *w, int N,
                            const Epi &epi, hipStream_t s) {
  const int tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
  const int grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_bf16_lds<Cfg, Epi, true>), dim3(grid), dim3(Cfg::NT), 0, s, o, w, M, N,
                     ns.Wa + ns.D, epi, ns);
  return hipGetLastError();
}

template <class Epi>
static hipError_t run_fused_auto(const bf16 *o, const NormScale &ns, int M, const bf16 *w, int N,
                                 const Epi &epi, hipStream_t s) {
  if (ns.Wa % CfgWide::BK == 0 && ns.D % CfgWide::BK == 0 && use_wide(M, N, ns.Wa + ns.D))
    return run_fused<CfgWide>(o, ns, M, w, N, epi, s);
  return run_fused<CfgLds>(o, ns, M, w, N, epi, s);
}

// (the y and o parts of K must each be whole k-tiles of the tile used)
bool outproj_fused_ok(int M, int Wa, int D) {
  static_assert(CfgWide::BK % CfgLds::BK == 0, "the deeper k-tile is a multiple of the other");
  return M >= 1024 && Wa > 0 && D > 0 && Wa % CfgLds::BK == 0 && D % CfgLds::BK == 0;
}

template <>
hipError_t launch_outproj_fused<bf16>(const bf16 *o, const NormScale &ns, int M, const bf16 *w, int Ncols,
                                      bf16 *out, const bf16 *resid, hipStream_t s) {
  if (!outproj_fused_ok(M, ns.Wa, ns.D)) return hipErrorInvalidValue;
  if (resid) return run_fused_auto(o, ns, M, w, Ncols, ResidEpi<bf16>{out, resid, Ncols}, s);
  return run_fused_auto(o, ns, M, w, Ncols, StoreEpi<bf16>{out, Ncols}, s);
}
template <>
hipError_t launch_outproj_fused<float>(const float *, const NormScale &, int, const float *, int, float *,
                                       const float *, hipStream_t) {
  return hipErrorInvalidValue;   // the fp32 path keeps the separate norm kernel
}

size_t skinny_part_bytes(int M, int K, int N) {
  if (M >= 1024) return 0;
  const int splits = skinny_splits(M, K, N);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

template <class Epi>
static hipError_t run_f32(const float *A, int M, int K, const float *B, int N, const Epi &epi,
                          hipStream_t s) {
  if (N % 4) return hipErrorInvalidValue;   // epilogue groups of 4 columns
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_tiled<Epi>), grid, dim3(256), 0, s, A, B, M, N, K, epi);
  return hipGetLastError();
}

template <>
hipError_t launch_inproj<bf16>(const bf16 *x, int M, int K, const bf16 *w, int Ncols,
                               const InProjOut &e, float *part, hipStream_t s) {
  if (e.rope_base == 0.0f) return run_bf16_auto(x, M, K, w, Ncols, InProjEpi<bf16, ROPE_NONE>{e}, part, s);
  // RoPE: the 256x256 tile's lanes own both halves of their pairs when a
  // wave's 64 columns are one head; the few-row tile reads the weight rows in
  // pair order instead, and is not split over K (the partial GEMMs would not
  // see that order)
  if (M >= 1024 && e.hd == CfgLds::WN)
    return run_lds<CfgLds>(x, M, K, w, Ncols, InProjEpi<bf16, ROPE_SPLIT_GROUPS>{e}, s);
  if (M >= 1024) return run_lds<CfgLds>(x, M, K, w, Ncols, InProjEpi<bf16, ROPE_PAIRED_COLS>{e}, s);
  return run_skinny(x, M, K, w, Ncols, InProjEpi<bf16, ROPE_PAIRED_COLS>{e}, nullptr, s);
}
template <>
hipError_t launch_inproj<float>(const float *x, int M, int K, const float *w, int Ncols,
                                const InProjOut &e, float *, hipStream_t s) {
  if (e.rope_base != 0.0f) return run_f32(x, M, K, w, Ncols, InProjEpi<float, ROPE_PAIRED_COLS>{e}, s);
  return run_f32(x, M, K, w, Ncols, InProjEpi<float, ROPE_NONE>{e}, s);
}
template <>
hipError_t launch_outproj<bf16>(const bf16 *f, int M, int K, const bf16 *w, int Ncols, bf16 *out,
                                const bf16 *resid, float *part, hipStream_t s) {
  if (resid) return run_bf16_auto(f, M, K, w, Ncols, ResidEpi<bf16>{out, resid, Ncols}, part, s);
  return run_bf16_auto(f, M, K, w, Ncols, StoreEpi<bf16>{out, Ncols}, part, s);
}
template <>
hipError_t launch_outproj<float>(const float *f, int M, int K, const float *w, int Ncols,
                                 float *out, const float *resid, float *, hipStream_t s) {
  if (resid) return run_f32(f, M, K, w, Ncols, ResidEpi<float>{out, resid, Ncols}, s);
  return run_f32(f, M, K, w, Ncols, StoreEpi<float>{out, Ncols}, s);
}
template <>
hipError_t launch_mlp_gate_up<bf16>(const bf16 *x, int M, int K, const bf16 *w, int Ncols,
                                    bf16 *h, float *part, hipStream_t s) {
  if (Ncols % 8) return hipErrorInvalidValue;
  return run_bf16_auto(x, M, K, w, Ncols, GluEpi<bf16>{h, Ncols / 2}, part, s);
}
template <>
hipError_t launch_mlp_gate_up<float>(const float *x, int M, int K, const float *w, int Ncols,
                                     float *h, float *, hipStream_t s) {
  if (Ncols % 8) return hipErrorInvalidValue;
  return run_f32(x, M, K, w, Ncols, GluEpi<float>{h, Ncols / 2}, s);
}

}  // namespace hh

// The attention heads and the SSM heads' scan pass 3 in one launch.
//
// The two branches of the hybrid-head layer (Hymba paper §2.1, Eqs. (1) and
// (2)) are independent once the input projection and the scan's chunk carries
// exist; the authors' reply on parallel computation notes that running them
// truly in parallel needs a kernel of its own.  Two kernels on two streams do
// not share CUs well (the first grid fills every CU and the second runs in
// its tail), so here one grid holds both kinds of workgroup, spread evenly
// over the block ids, and every CU runs attention and scan waves side by side
// from start to end.  It is an opt-in path (HH_ONE_LAUNCH_BRANCHES=1):
// measured on the 8k prefill it takes about as long as the two kernels one
// after the other (245-250 us against 117 + 125 us).  Each kernel alone fills
// a CU's registers and LDS and hides latency with its wave count, and the
// scan's VALU work plus the softmax's exceed the VALU issue rate, so sharing
// the CUs only divides them.
//
// A workgroup has NW waves.  Attention role: exactly the attention kernel's
// workgroup (attn_body.inc).  Scan role: its first min(NW, 4) waves each run
// pass 3 for one 64-channel block of one chunk (scan_dev.h), with LDS borrowed
// from the attention's arrays (B|C staging in four 8 KB stage arrays, the row
// sums' tables in the other two); the other waves end at once.
#include "attn_dev.h"
#include "scan_dev.h"

namespace hh {

namespace {

constexpr int kScanWavesMax = 4;   // scan waves per workgroup (four 8 KB B|C buffers)

template <int NW, class T, bool SC, int OUT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
attn_scan3(AttnArgs aa, ScanArgs sa, int n_attn, int n_scan) {
#if defined(__HIP_DEVICE_COMPILE__)
  using namespace adev;
  __shared__ uint4 sK0[TILE_UNITS], sK1[TILE_UNITS], sK2[TILE_UNITS];
  __shared__ uint4 sV0[TILE_UNITS], sV1[TILE_UNITS], sV2[TILE_UNITS];
  __shared__ float sq_part[NW][32];
  __shared__ float sbeta[NW * HD];
  // block i is a scan workgroup when the count of scan workgroups among ids
  // [0, i] exceeds that among [0, i): the roles interleave evenly
  const long total = (long)n_attn + n_scan;
  const long i = blockIdx.x;
  const int s_before = (int)(i * n_scan / total), s_upto = (int)((i + 1) * n_scan / total);
  if (s_upto > s_before) {
    constexpr int SW = NW < kScanWavesMax ? NW : kScanWavesMax;
    static_assert(sdev::SUB * 2 * sdev::NS * 4 == sizeof(sK0), "one stage array per scan wave");
    static_assert(3 * sdev::TB * sdev::SQ_LD * 4 <= (int)sizeof(sK0), "three row-sum tables per array");
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (wave >= SW) return;
    const int nc = (sa.n + sa.chunk - 1) / sa.chunk;
    const int ncb = (sa.D + 63) / 64, ncg = (ncb + SW - 1) / SW;
    const int si = s_before;
    const int ck = si % nc, cg = (si / nc) % ncg, b = si / (nc * ncg);
    const int cb = cg * SW + wave;
    if (cb >= ncb) return;
    float *sbc = reinterpret_cast<float *>(wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sK2 : sV0);
    float *sq = wave < 3 ? reinterpret_cast<float *>(sV1) + wave * (sdev::TB * sdev::SQ_LD)
                         : reinterpret_cast<float *>(sV2);
    sdev::pass3_wave<T, SC, OUT>(sa, ck, cb, b, sbc, sq);
    return;
  }
  const int ai = (int)i - s_before;
  const int nqt_all = (aa.n + BQ - 1) / BQ;
  const int bx = ai % nqt_all, g = (ai / nqt_all) % aa.G, b = ai / (nqt_all * aa.G);
  const AttnArgs &a = aa;
#include "attn_body.inc"
#endif
}

template <int NW, bool SC, int OUT>
hipError_t launch_nw(const AttnArgs &aa, const ScanArgs &sa, hipStream_t s) {
  constexpr int SW = NW < kScanWavesMax ? NW : kScanWavesMax;
  const int nqt = (aa.n + adev::BQ - 1) / adev::BQ;
  const int n_attn = nqt * aa.G * aa.B;
  const int nc = (sa.n + sa.chunk - 1) / sa.chunk;
  const int ncg = ((sa.D + 63) / 64 + SW - 1) / SW;
  const int n_scan = nc * ncg * sa.B;
  hipLaunchKernelGGL((attn_scan3<NW, bf16, SC, OUT>), dim3(n_attn + n_scan), dim3(NW * 64), 0, s, aa, sa,
                     n_attn, n_scan);
  return hipGetLastError();
}

template <bool SC, int OUT>
hipError_t launch_mode(const AttnArgs &aa, const ScanArgs &sa, hipStream_t s) {
  switch (aa.H / aa.G) {
    case 1: return launch_nw<1, SC, OUT>(aa, sa, s);
    case 2: return launch_nw<2, SC, OUT>(aa, sa, s);
    case 3: return launch_nw<3, SC, OUT>(aa, sa, s);
    case 4: return launch_nw<4, SC, OUT>(aa, sa, s);
    case 5: return launch_nw<5, SC, OUT>(aa, sa, s);
    case 6: return launch_nw<6, SC, OUT>(aa, sa, s);
    case 7: return launch_nw<7, SC, OUT>(aa, sa, s);
    case 8: return launch_nw<8, SC, OUT>(aa, sa, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

template <>
hipError_t launch_attn_scan3<bf16>(const AttnArgs &aa, const ScanArgs &sa, hipStream_t s) {
  const int mode = sdev::pass3_mode(sa);
  if (mode == 3) return hipErrorInvalidValue;   // the prefill always writes Y
  if (sa.S) return mode == 2 ? launch_mode<true, 2>(aa, sa, s) : launch_mode<true, 1>(aa, sa, s);
  return mode == 2 ? launch_mode<false, 2>(aa, sa, s) : launch_mode<false, 1>(aa, sa, s);
}

template <>
hipError_t launch_attn_scan3<float>(const AttnArgs &, const ScanArgs &, hipStream_t) {
  return hipErrorInvalidValue;   // the fp32 attention has its own kernel
}

}  // namespace hh

// Device code of the bf16 prefill attention, shared by the attention
// kernel and the launch that runs it beside scan pass 3 (the method is
// described in attention.hip).
#pragma once
#include "hh_internal.h"

namespace hh {
namespace adev {

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

// K and V tiles are streamed into LDS as they lie in memory (64 keys x 128 B,
// 16-byte chunks XOR-swizzled per row) by buffer_load ... lds, STAGES tiles
// deep.  The V^T operand of O^T = V^T P^T is read with ds_read_b64_tr_b16:
// inside each 16-lane group, lane j receives element j%4 of the 8-byte loads
// addressed by lanes 4k + j/4 (k = 0..3), so lane l addressing key row
// 16ks + 4(l/32) + (l%16)/4 (+8) and columns 32dblk + 16((l/16)%2) + 4(l%4)
// hands every lane the 4 consecutive keys of its own d = 32dblk + l%32.
constexpr int ASTAGES = 3;
constexpr int TILE_UNITS = BKV * HD / 8;     // 512 16-byte units per K (or V) tile
// the body of a workgroup (attn_body.inc) is expanded inside each kernel
// that runs one, with these LDS arrays declared in that kernel

}  // namespace adev
}  // namespace hh

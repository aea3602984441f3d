// Device helpers shared by the KVarN HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kDim = 128;         // head_dim = channels per tile
constexpr int kTile = 128;        // tokens per tile / page
constexpr int kKRecord = 9216;    // bytes of a key page record
constexpr int kVRecord = 5120;    // bytes of a value page record
constexpr int kKCodeBytes = 8192; // 4-bit codes of a key record
constexpr int kK2Record = 5120;   // bytes of a 2-bit key page record (preset kvarn_k2v2_g128)
constexpr int kK2CodeBytes = 4096; // 2-bit codes of such a record
constexpr int kV4Record = 9216;   // bytes of a 4-bit value page record (preset kvarn_k4v4_g128)
constexpr int kV4CodeBytes = 8192; // 4-bit codes of such a record
constexpr int kVCodeBytes = 4096; // 2-bit codes of a value record
constexpr float kInvSqrt128 = 0.08838834764831845f;  // 1 / sqrt(128), fp32-rounded

// Float16 metadata after a record's codes, in slots of 128 values: format 1 holds r, s, then
// the group scales and zeros; format 2 (folded) holds the normalizer of the other axis, then
// the scales and zeros with the group's own normalizer folded in (keys s, scale', zero' per
// channel, of Xr / s; values r, scale', zero' per token, of Xr / r). NG groups per key channel
// or value token: 1 (group 128: one scale slot, one zero slot) or 2 (group 64: the scales of
// halves 0 and 1, then the zeros of halves 0 and 1; half 0 = tokens 0..63 of a key channel,
// channels 0..63 of a value token).
template <int FMT> constexpr int norm_slots() { return FMT == 1 ? 2 : 1; }
template <int FMT, int NG> constexpr int meta_slots() { return norm_slots<FMT>() + 2 * NG; }
template <int FMT, int NG> constexpr int meta_bytes() { return 256 * meta_slots<FMT, NG>(); }
template <int FMT, int NG> constexpr int slot_scale(int h) { return norm_slots<FMT>() + h; }
template <int FMT, int NG> constexpr int slot_zero(int h) { return norm_slots<FMT>() + NG + h; }
constexpr int kMaxMetaSlots = 6;

// ---- cross-lane moves -------------------------------------------------------------
// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRowRor8 = 0x128;      // rotate right by 8 inside a 16-lane row (= xor 8)

// Every control used here reads a lane inside the same 16-lane row, so no lane ever falls
// back to the bound value; bound_ctrl lets the compiler fold the move into the consumer.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// ds_swizzle in bit mode: lane l reads lane ((l & 0x1F) ^ XOR) within its 32-lane half.
template <int XOR>
__device__ __forceinline__ float swz_xor_f(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (XOR << 10)));
}

__device__ __forceinline__ float shfl_xor32_f(float v) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane ^ 32) << 2), __float_as_int(v)));
}

// Value of lane (l ^ m) for m in {1, 2, 4, 8} (stays inside the 16-lane row).
template <int M>
__device__ __forceinline__ float xor_lane16(float v) {
  if constexpr (M == 1) return dpp_f<kDppQuadXor1>(v);
  else if constexpr (M == 2) return dpp_f<kDppQuadXor2>(v);
  else if constexpr (M == 4) return swz_xor_f<4>(v);
  else return dpp_f<kDppRowRor8>(v);
}

// Sum over the 16 lanes of a row, result in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppRowRor8>(v);
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_f<kDppQuadXor1>(v));
  v = fminf(v, dpp_f<kDppQuadXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  v = fminf(v, dpp_f<kDppRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowRor8>(v));
  return v;
}

// Combine lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave).
__device__ __forceinline__ float rows4_sum(float v) {
  v += swz_xor_f<16>(v);
  v += shfl_xor32_f(v);
  return v;
}
__device__ __forceinline__ float rows4_min(float v) {
  v = fminf(v, swz_xor_f<16>(v));
  v = fminf(v, shfl_xor32_f(v));
  return v;
}
__device__ __forceinline__ float rows4_max(float v) {
  v = fmaxf(v, swz_xor_f<16>(v));
  v = fmaxf(v, shfl_xor32_f(v));
  return v;
}

// ---- float16 ----------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h_rn(float f) { return __half_as_ushort(__float2half_rn(f)); }

}  // namespace kvarn

// KVarN tile quantizer for gfx950.
//
// One workgroup (256 threads, 4 waves) quantizes one 128-token x 128-channel tile of one
// KV head (KVarN README, "How KVarN works", stages 1-4):
//   1. gather the float16 tile (channels x tokens) from a token-major stream;
//   2. rotate along channels, Xr = H X (H = normalized natural-order Sylvester Hadamard);
//   3. iterative log-space Sinkhorn-style normalization: each iteration sets every token's
//      normalizer s_t to the std over channels of Xr[:, t] / r, then every channel's r_c to
//      the std over tokens of Xr[c, :] / s (population std, centred; a zero std leaves the
//      normalizer unchanged). Accumulating log-std's as the pages describe telescopes to
//      exactly this assignment, so the kernel keeps 1/r, 1/s (rsqrt of the variances);
//   4. r, s rounded to float16; Y = Xr / (r s^T) against the stored values; asymmetric
//      round-to-nearest: keys 4-bit, one (scale, zero) per channel; values 2-bit, one per
//      token; codes packed in the page format of include/kvarn.h.
//
// Thread layout: thread (wave w, lane l) owns channels 8cb..8cb+7 (cb = l % 16) of 8 tokens,
// slot j holding token 32w + 16 (j / 4) + 4 (l / 16) + j % 4. That is the accumulator layout
// of the matrix-core rotation: the rotation is the dense product X H on the MFMA pipe
// (16x16x32 float16 blocks, +-1 entries, float32 accumulation), A = the raw float16 rows as
// loaded, B = H generated in registers, and the output columns are ordered so that a lane's
// 8 columns are 8 consecutive channels. Reductions over channels stay inside a 16-lane row
// (DPP); reductions over tokens combine the 4 rows of a wave (row-pair swaps) and the 4
// waves through LDS. Both are reduce-scatters: each group's statistic lands on one owner
// lane, which computes the group's weight once and broadcasts it back through LDS. The tile
// stays in registers (64 fp32 / thread). Key codes are packed in registers (a thread's 8
// channels of one token are one record word); value codes go through LDS.
#include "kvarn_device.h"
#include "kvarn_launch.h"

// Sums and products below are written in the order the numerics need; no contraction.
#pragma clang fp contract(off)

namespace kvarn {
namespace {

constexpr int kThreads = 256;

// Value codes are staged in LDS as one 128-byte row of token codes per channel. Row c starts at
// dword 36 c + 2 (c >> 3): the 32 lanes of one pass of a 4-byte write (16 channel blocks, two
// token groups) and of the packing reads (4 channels, 4 token groups, 2 steps) then fall into
// 32 distinct banks. A stride of 32 dwords puts all 16 channel blocks in one bank.
constexpr int kCodeRowBase = 36;
__device__ __forceinline__ int codes_row(int c) { return kCodeRowBase * c + 2 * (c >> 3); }

struct QuantSmem {
  float red[2][4][kDim];       // per-wave partial sums over tokens, channel vectors (2 buffers)
  float gr[4][2][kDim];        // per-wave broadcast of channel vectors (chan_pair_slot order)
  float gc[4][4][2][2][8];     // per-wave, per-row, per-half broadcast of per-token values
  uint32_t codes[kCodeRowBase * kDim + 2 * 16];  // value codes: row c at codes_row(c)
  uint16_t meta[kMaxMetaSlots][kDim];  // the record's metadata slots as float16 bits
};

constexpr int kDppRowRor4 = 0x124;  // rotate right by 4 inside a 16-lane row

template <int OP>  // 0 sum, 1 min, 2 max
__device__ __forceinline__ float combine(float a, float b) {
  if constexpr (OP == 0) return a + b;
  else if constexpr (OP == 1) return fminf(a, b);
  else return fmaxf(a, b);
}

// Reduce-scatter over the 16 lanes of a row: every lane holds v[0..7] (one value per token
// of its token block); lane l returns the row-wide reduction of v[l & 7] (lanes l and l ^ 8
// agree); with FULL = false, the reduction over the 8 lanes whose bit 3 equals l's. Each stage keeps the half of the values whose index bit matches the lane bit and
// adds the partner's copy of that half: bits 0 and 1 with quad permutes, bit 2 with a
// rotation by 4 (any partner with the other bit 2 works, since bit 3 is summed last).
template <int OP, bool FULL = true>
__device__ __forceinline__ float row16_scatter8(const float (&v)[8], int l) {
  const bool b0 = (l & 1) != 0, b1 = (l & 2) != 0, b2 = (l & 4) != 0;
  float a[4], c[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float send = b0 ? v[2 * k] : v[2 * k + 1];
    const float keep = b0 ? v[2 * k + 1] : v[2 * k];
    a[k] = combine<OP>(keep, dpp_f<kDppQuadXor1>(send));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float send = b1 ? a[2 * k] : a[2 * k + 1];
    const float keep = b1 ? a[2 * k + 1] : a[2 * k];
    c[k] = combine<OP>(keep, dpp_f<kDppQuadXor2>(send));
  }
  const float send = b2 ? c[0] : c[1];
  const float keep = b2 ? c[1] : c[0];
  if constexpr (!FULL) {
    // partner exactly lane l ^ 4 (a rotation by 4 would pair lanes 0..3 with 12..15, across
    // the halves): the reduction stays inside the 8 lanes whose bit 3 equals l's
    return combine<OP>(keep, swz_xor_f<4>(send));
  }
  const float e = combine<OP>(keep, dpp_f<kDppRowRor4>(send));
  return combine<OP>(e, dpp_f<kDppRowRor8>(e));
}

// Reduce-scatter over the 4 rows of a wave with the row-pair swaps of gfx950: every lane
// holds v[0..7] (one value per channel of its channel block); a lane of row r returns the
// reduction over the 4 rows of v[k + off(r)], k = 0, 1, off(r) = 4 (r & 1) + 2 (r >> 1).
template <int OP>
__device__ __forceinline__ void rows4_scatter8(const float (&v)[8], float (&o)[2]) {
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]),
                                                    false, false);
    u[i] = combine<OP>(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(u[i]), __float_as_uint(u[i + 2]),
                                                    false, false);
    o[i] = combine<OP>(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
}

__device__ __forceinline__ void lds_read8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Per-channel float vectors in LDS (128 floats): channel 8 cb + o lives at float
// 64 (o >> 2) + 4 cb + ((o & 3) ^ 2 (o >> 2)). The two channels an owner lane holds
// (o = off, off + 1 with off even) are one aligned float2, and a lane's block of 8 channels is
// two float4 loads; the float2 stores of a 16-lane pass hit distinct bank pairs except for one
// 2-way overlap, where channel-major order (a 32-byte stride) costs 4-way conflicts on the
// stores and 2-way ones on the block loads.
__device__ __forceinline__ int chan_pair_slot(int cb, int off) {
  return 64 * (off >> 2) + 4 * cb + ((off & 3) ^ (2 * (off >> 2)));
}
__device__ __forceinline__ void chan_read8(const float* p, int cb, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p + 4 * cb);        // o = 0, 1, 2, 3
  const float4 b = *reinterpret_cast<const float4*>(p + 64 + 4 * cb);   // o = 6, 7, 4, 5
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.z; v[5] = b.w; v[6] = b.x; v[7] = b.y;
}

// float16 bits of a normalizer: clipped to [2^-14, 65504] first
__device__ __forceinline__ uint16_t normalizer16(float v) {
  return f2h_rn(fminf(fmaxf(v, 6.103515625e-05f), 65504.f));
}
// float16 bits of a scale or zero point: saturated to the finite range [-65504, 65504] first
// (a near-constant group can normalize to values beyond float16; the record stays finite)
__device__ __forceinline__ uint16_t meta16(float v) {
  return f2h_rn(fminf(fmaxf(v, -65504.f), 65504.f));
}

// 4 codes (bytes, each <= 3) -> 4 crumbs in the low 8 bits, byte k -> crumb k
__device__ __forceinline__ uint32_t bytes_to_crumbs(uint32_t e) {
  const uint32_t x = (e | (e >> 6)) & 0x000F000Fu;
  return (x | (x >> 12)) & 0x000000FFu;
}

// Record geometry by kind and code width (presets kvarn_k4v2_g128, kvarn_k2v2_g128,
// kvarn_k4v4_g128).
template <int KIND, int BITS> struct CodeBytes;
template <> struct CodeBytes<0, 4> { static constexpr int kBytes = kKCodeBytes; };
template <> struct CodeBytes<0, 2> { static constexpr int kBytes = kK2CodeBytes; };
template <> struct CodeBytes<1, 2> { static constexpr int kBytes = kVCodeBytes; };
template <> struct CodeBytes<1, 4> { static constexpr int kBytes = kV4CodeBytes; };
// FMT 1: codes, then r, s, scale, zero; FMT 2 (folded): codes, then keys s, scale', zero' /
// values r, scale', zero'
template <int KIND, int BITS, int FMT, int NG> struct RecFormat {
  static constexpr int kCodeBytes = CodeBytes<KIND, BITS>::kBytes;
  static constexpr int kRecord = kCodeBytes + meta_bytes<FMT, NG>();
};

// x += c * x(lane under DPP control CTRL) for 8 values, one v_fmac_f32_dpp each. The DPP
// source is read from the register the instruction writes (all lanes read before any
// writes). A DPP read of a VGPR needs 2 wait states after the VALU write of that VGPR: the
// block starts with them (s_nop 1), and no instruction of the block reads a value written
// inside it. bound_ctrl is irrelevant: every control used reads inside the 16-lane row.
#define KVARN_FMAC_DPP8(CTRL, C, X)                                                         \
  asm volatile("s_nop 1\n"                                                                   \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"     \
               : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3]), "+v"(X[4]), "+v"(X[5]),   \
                 "+v"(X[6]), "+v"(X[7])                                                     \
               : "v"(C))

// FWHT stages after the first (channel bit 0): bits 1, 2 in-thread, bits 3..6 = lane bits
// 0..3, then * 1/sqrt(128). A cross-lane stage on lane bit m is one fused multiply-add per
// value: y += c * y(lane ^ m) with c = +1 on lanes whose bit m is 0 and -1 on the others.
// Lanes with the bit set then hold the negated difference; the accumulated sign,
// (-1)^popcount(lane bits 0..3), is removed by the final scaling.
__device__ __forceinline__ void fwht_after_first(float (&x)[8][8], int cb) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int h = 2; h < 8; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((i & h) == 0) {
          float a = x[j][i], b = x[j][i + h];
          x[j][i] = a + b;
          x[j][i + h] = a - b;
        }
      }
    }
  }
  const float c1 = (cb & 1) ? -1.f : 1.f, c2 = (cb & 2) ? -1.f : 1.f;
  const float c4 = (cb & 4) ? -1.f : 1.f, c8 = (cb & 8) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) KVARN_FMAC_DPP8("quad_perm:[1,0,3,2]", c1, x[j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) KVARN_FMAC_DPP8("quad_perm:[2,3,0,1]", c2, x[j]);
  // lane bit 2: ds_swizzle (xor 4 is not a DPP row pattern); partners of one token's 8
  // values are fetched before any of them is updated
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = swz_xor_f<4>(x[j][i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[j][i] = fmaf(p[i], c4, x[j][i]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) KVARN_FMAC_DPP8("row_ror:8", c8, x[j]);
  const float fin = (__builtin_popcount(cb) & 1) ? -kInvSqrt128 : kInvSqrt128;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[j][i] *= fin;
}

// The same transform on float32 values.
__device__ __forceinline__ void fwht_channels_f32(float (&x)[8][8], int cb) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = x[j][2 * k], b = x[j][2 * k + 1];
      x[j][2 * k] = a + b;
      x[j][2 * k + 1] = a - b;
    }
  }
  fwht_after_first(x, cb);
}
#undef KVARN_FMAC_DPP8

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
union H8 {
  half8 v;
  uint32_t u[4];
};

// Dword d (elements 2d, 2d+1) of the Walsh pattern (-1)^popcount(i & c), i = 0..7, as
// float16 +-1: the within-block part of the Hadamard column block c.
__host__ __device__ constexpr uint32_t walsh8_dword(int c, int d) {
  uint32_t w = 0;
  for (int e = 0; e < 2; ++e) {
    const int i = 2 * d + e;
    int par = 0;
    for (int b = i & c; b; b >>= 1) par ^= b & 1;
    w |= uint32_t(par ? 0xBC00u : 0x3C00u) << (16 * e);
  }
  return w;
}

// Rotation X -> X H of the wave's 32 tokens on the matrix cores, H the natural-order
// Sylvester matrix with entries +-1: the result is sqrt(128) times the orthonormal rotation
// (the factor is carried by the channel weights of the normalization, see quantize_tile). MFMA block (token block tb2, input channels
// 32 kb .. 32 kb + 31) x (those channels, output column block cc): A lane l = token
// 32w + 16 tb2 + l % 16, input channels 32 kb + 8 (l / 16) + i (one 16-byte load); B lane
// l = the same input channels, output channel 8 (l % 16) + cc. The sign of H at (input a,
// output b) is (-1)^popcount(a & b), which splits into the Walsh pattern of i & cc
// (a compile-time constant per cc) and a per-lane sign (-1)^popcount((4 kb + l / 16) &
// (l % 16)) applied by one XOR per dword. Accumulator element r of block (tb2, cc) is token
// slot 4 tb2 + r, channel 8 (l % 16) + cc.
template <typename RowPtr>
__device__ __forceinline__ void rotate_tile_mfma(RowPtr row_ptr, int w, int l, float (&x)[8][8]) {
  const int q = l >> 4, m = l & 15;
  H8 a[2][4];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const __half* row = row_ptr(32 * w + 16 * t2 + m);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + 32 * kb + 8 * q);
      a[t2][kb].u[0] = v.x; a[t2][kb].u[1] = v.y; a[t2][kb].u[2] = v.z; a[t2][kb].u[3] = v.w;
    }
  }
  uint32_t sgn[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    sgn[kb] = (__builtin_popcount((4 * kb + q) & m) & 1) ? 0x80008000u : 0u;
  // k-step outermost: the 16 accumulators are the tile itself, each one's 4 products are
  // 16 MFMAs apart, and a k-step's A fragments die after it
  float4v acc[2][8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    acc[0][cc] = float4v{0.f, 0.f, 0.f, 0.f};
    acc[1][cc] = float4v{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      H8 b;
#pragma unroll
      for (int d = 0; d < 4; ++d) b.u[d] = walsh8_dword(cc, d) ^ sgn[kb];
      acc[0][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0][kb].v, b.v, acc[0][cc], 0, 0, 0);
      acc[1][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1][kb].v, b.v, acc[1][cc], 0, 0, 0);
    }
    // keep each k-step's B fragments inside it (register pressure)
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r][cc] = acc[0][cc][r];
      x[4 + r][cc] = acc[1][cc][r];
    }
}

// The tile quantizer proper. row_ptr(t) gives the 16-byte aligned address of token t's
// 128 channels. Writes one record at `rec`; BITS is the code width of this kind.
template <int KIND, int BITS, int FMT, int NG, typename RowPtr>
__device__ __forceinline__ void quantize_tile(RowPtr row_ptr, uint8_t* __restrict__ rec, int n_iters,
                                              QuantSmem& sm) {
  // metadata slots of the record: format 1 r, s, then scales and zeros; format 2 the other
  // axis's normalizer, then scales' and zeros' (the group's normalizer folded in); NG = 2
  // (group 64) has a scale and a zero slot per half (slot_scale / slot_zero)
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int cb = l & 15;
  // token of slot j (the rotation's accumulator layout)
  auto tok = [&](int j) { return 32 * w + 16 * (j >> 2) + 4 * (l >> 4) + (j & 3); };

  // ---- 1-2. gather and rotate: x[j][i] = sqrt(128) (H X)[8cb + i, token of slot j] ---------
  // x is kept unnormalized: the channel weights below start at 1/sqrt(128) instead of 1, so
  // every channel variance (and r) is computed 128 (sqrt(128)) times too large, which the
  // stored r and the code factors undo exactly (a power of two) or once per group.
  float x[8][8];
  rotate_tile_mfma(row_ptr, w, l, x);

  // ---- 3. normalize -----------------------------------------------------------------
  // Two passes per step (mean, then centred sum of squares), float32 FMAs. A group's
  // statistics are reduce-scattered to one owner lane: token slot l & 7 for the column
  // step (over channels), channels 8 cb + off + {0, 1} for the row step (over tokens; the
  // 4 waves add their partials through LDS); the owner computes the group's weight and LDS
  // broadcasts it back inside the wave. The next step's weights are 1/std = rsqrt(var). A
  // group whose variance is below 1e-12 mean^2 is constant up to float32 rounding (a
  // non-constant group of float16-derived values has a relative spread of at least ~1e-5):
  // its update is skipped, as for an exactly zero std.
  const int r = l >> 4;
  const int tok_own = l & 7;
  const int ch_off = 4 * (r & 1) + 2 * (r >> 1);
  const int ch_own = 8 * cb + ch_off;
  const int own_slot = chan_pair_slot(cb, ch_off);  // my channel pair in a channel vector
  float* gc0 = &sm.gc[w][r][0][0][0];
  float* gr0 = &sm.gr[w][0][0];
  float ir[8], is[8];      // 1/r for my channels, 1/s for my tokens
#pragma unroll
  for (int i = 0; i < 8; ++i) { ir[i] = kInvSqrt128; is[i] = 1.f; }
  float vs_own = 1.f;                  // last accepted variance of my token (1 = never)
  float vr_own[2] = {128.f, 128.f};    // ... of my two channels, in units of x (128 = never)
  int buf = 0;
  auto cross_wave_sum = [&](const float (&o)[2], float (&t)[2]) {
    *reinterpret_cast<float2*>(&sm.red[buf][w][own_slot]) = make_float2(o[0], o[1]);
    __syncthreads();
    float2 a = *reinterpret_cast<const float2*>(&sm.red[buf][0][own_slot]);
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      const float2 b = *reinterpret_cast<const float2*>(&sm.red[buf][ww][own_slot]);
      a.x += b.x;
      a.y += b.y;
    }
    t[0] = a.x;
    t[1] = a.y;
    buf ^= 1;
  };
  for (int it = 0; it < n_iters; ++it) {
    // column step: per token, over the 128 channels
    float m[8], q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = x[j][0] * ir[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) a = fmaf(x[j][i], ir[i], a);
      m[j] = a;
    }
    const float mean_t = row16_scatter8<0>(m, l) * (1.f / kDim);
    gc0[tok_own] = -mean_t;
    lds_read8(gc0, m);                       // minus the means of my 8 tokens
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = fmaf(x[j][i], ir[i], m[j]);
        a = fmaf(d, d, a);
      }
      q[j] = a;
    }
    {
      const float var = row16_scatter8<0>(q, l) * (1.f / kDim);
      vs_own = var > 1e-12f * mean_t * mean_t ? var : vs_own;
      gc0[tok_own] = __builtin_amdgcn_rsqf(vs_own);
      lds_read8(gc0, is);
    }
    // row step: per channel, over the 128 tokens
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = x[0][i] * is[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) a = fmaf(x[j][i], is[j], a);
      m[i] = a;
    }
    float o[2], mean_c[2];
    rows4_scatter8<0>(m, o);
    cross_wave_sum(o, mean_c);
    mean_c[0] *= 1.f / kTile;
    mean_c[1] *= 1.f / kTile;
    *reinterpret_cast<float2*>(&gr0[own_slot]) = make_float2(-mean_c[0], -mean_c[1]);
    chan_read8(gr0, cb, m);             // minus the means of my 8 channels
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = fmaf(x[j][i], is[j], m[i]);
        a = fmaf(d, d, a);
      }
      q[i] = a;
    }
    float var_c[2];
    rows4_scatter8<0>(q, o);
    cross_wave_sum(o, var_c);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float var = var_c[k] * (1.f / kTile);
      vr_own[k] = var > 1e-12f * mean_c[k] * mean_c[k] ? var : vr_own[k];
    }
    *reinterpret_cast<float2*>(&gr0[own_slot]) =
        make_float2(__builtin_amdgcn_rsqf(vr_own[0]), __builtin_amdgcn_rsqf(vr_own[1]));
    chan_read8(gr0, cb, ir);
  }

  // ---- 4a. stored normalizers (float16) and their inverses on every lane ----------------
  const uint16_t s16 = normalizer16(__builtin_amdgcn_sqrtf(vs_own));
  const uint16_t r16a = normalizer16(__builtin_amdgcn_sqrtf(vr_own[0] * (1.f / 128.f)));
  const uint16_t r16b = normalizer16(__builtin_amdgcn_sqrtf(vr_own[1] * (1.f / 128.f)));
  const float is_own = __builtin_amdgcn_rcpf(h2f(s16));
  // 1 / (sqrt(128) r): divides x (unnormalized) by the stored r
  const float ir_own[2] = {__builtin_amdgcn_rcpf(h2f(r16a)) * kInvSqrt128,
                           __builtin_amdgcn_rcpf(h2f(r16b)) * kInvSqrt128};
  if (FMT == 1 || KIND == 1) {
    if (w == 0) {            // every channel once
      sm.meta[0][ch_own] = r16a;
      sm.meta[0][ch_own + 1] = r16b;
    }
  }
  if (FMT == 1 || KIND == 0) {
    if ((l & 8) == 0) sm.meta[FMT == 1 ? 1 : 0][tok(tok_own)] = s16;   // every token once
  }
  gc0[tok_own] = is_own;
  lds_read8(gc0, is);
  *reinterpret_cast<float2*>(&gr0[own_slot]) = make_float2(ir_own[0], ir_own[1]);
  chan_read8(gr0, cb, ir);

  // ---- 4b. asymmetric RTN --------------------------------------------------------------
  // code = clamp(rne((y - zero) / scale), 0, top) with y = x / (r s): computed as
  // fma(z, A, B), z the element times one of its two inverse normalizers and A, B per group;
  // cvt_pk_u8 rounds to nearest even and clamps below at 0, the min clamps above.
  uint32_t* out = reinterpret_cast<uint32_t*>(rec);
  if constexpr (KIND == 0) {
    // keys: one group per channel, over the 128 tokens; z = x / s
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[j][i] *= is[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn[i] = x[0][i];
      mx[i] = x[0][i];
#pragma unroll
      for (int j = 1; j < 8; ++j) { mn[i] = fminf(mn[i], x[j][i]); mx[i] = fmaxf(mx[i], x[j][i]); }
    }
    float omn[2], omx[2];
    rows4_scatter8<1>(mn, omn);
    rows4_scatter8<2>(mx, omx);
    // the 4 waves' partials through the (free) broadcast area; both red buffers are free
    // once every thread is past this barrier
    *reinterpret_cast<float2*>(&sm.gr[w][0][own_slot]) = make_float2(omn[0], omn[1]);
    *reinterpret_cast<float2*>(&sm.gr[w][1][own_slot]) = make_float2(omx[0], omx[1]);
    __syncthreads();
    // NG = 2: a group is the 64 tokens of waves 2h, 2h + 1 (h = w / 2)
#pragma unroll
    for (int k2 = 0; k2 < 4 / NG; ++k2) {
      const int ww = NG == 1 ? k2 : (w & 2) + k2;
      const float2 a = *reinterpret_cast<const float2*>(&sm.gr[ww][0][own_slot]);
      const float2 b = *reinterpret_cast<const float2*>(&sm.gr[ww][1][own_slot]);
      omn[0] = fminf(omn[0], a.x); omn[1] = fminf(omn[1], a.y);
      omx[0] = fmaxf(omx[0], b.x); omx[1] = fmaxf(omx[1], b.y);
    }
    float A2[2], B2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // format 1: the group is y = z / r (r > 0); format 2 codes z = Xr / s itself (r folded
      // into the stored scale and zero); x carries sqrt(128)
      const float to_g = FMT == 1 ? ir_own[k] : kInvSqrt128;
      const float lo = omn[k] * to_g, hi_ = omx[k] * to_g;
      const uint16_t sc16 = meta16((hi_ - lo) * (BITS == 4 ? 1.f / 15.f : 1.f / 3.f));
      const uint16_t zr16 = meta16(lo);
      const float sc = h2f(sc16);
      const float inv = sc > 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;
      A2[k] = to_g * inv;
      B2[k] = -h2f(zr16) * inv;
      if ((w & (NG == 1 ? 3 : 1)) == 0) {   // one wave per group
        sm.meta[slot_scale<FMT, NG>(w >> 1 & (NG - 1))][ch_own + k] = sc16;
        sm.meta[slot_zero<FMT, NG>(w >> 1 & (NG - 1))][ch_own + k] = zr16;
      }
    }
    float* ga = &sm.red[0][w][0];
    float* gb = &sm.red[1][w][0];
    *reinterpret_cast<float2*>(&ga[own_slot]) = make_float2(A2[0], A2[1]);
    *reinterpret_cast<float2*>(&gb[own_slot]) = make_float2(B2[0], B2[1]);
    float A[8], B[8];
    chan_read8(ga, cb, A);
    chan_read8(gb, cb, B);
    if constexpr (BITS == 4) {
      // word (t, cb) = channels 8cb..8cb+7 of token t; nibble p <- channel {0,2,4,6,1,3,5,7}[p]:
      // channel i's code goes to byte i / 4 of register i % 4 (registers hold channels {0, 4},
      // {1, 5}, {2, 6}, {3, 7}); codes are at most 15, so shift-ors interleave them into nibbles
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t r[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u = fminf(fmaf(x[j][i], A[i], B[i]), 15.f);
          r[i & 3] = __builtin_amdgcn_cvt_pk_u8_f32(u, i >> 2, r[i & 3]);
        }
        const uint32_t lo = r[0] | (r[2] << 4);   // nibbles 0..3: channels 0, 2, 4, 6
        const uint32_t hi = r[1] | (r[3] << 4);   // nibbles 4..7: channels 1, 3, 5, 7
        out[tok(j) * 16 + cb] = lo | (hi << 16);
      }
    } else {
      // 2-bit keys: token t's word w = 2 g + d holds channel 32 g + 8 (2 d + hs) + 2 v + e in
      // crumb 4 hs + v + 8 e, i.e. channels 16 w .. 16 w + 15. This thread's 8 channels
      // (cb = 2 w + hs) fill crumbs 4 hs .. +3 (even channels) and 8 + 4 hs .. +3 (odd
      // channels); the thread with cb ^ 1 (lane l ^ 1) holds the other half of the word.
      const int hs = cb & 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t e = 0, o = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u = fminf(fmaf(x[j][i], A[i], B[i]), 3.f);
          if (i & 1) o = __builtin_amdgcn_cvt_pk_u8_f32(u, i >> 1, o);
          else e = __builtin_amdgcn_cvt_pk_u8_f32(u, i >> 1, e);
        }
        const uint32_t mine = (bytes_to_crumbs(e) | (bytes_to_crumbs(o) << 16)) << (8 * hs);
        const uint32_t other = __float_as_uint(dpp_f<kDppQuadXor1>(__uint_as_float(mine)));
        if (hs == 0) out[tok(j) * 8 + (cb >> 1)] = mine | other;
      }
    }
  } else {
    // values: one group per token, over the 128 channels; z = x / r
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[j][i] *= ir[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mn[j] = x[j][0];
      mx[j] = x[j][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) { mn[j] = fminf(mn[j], x[j][i]); mx[j] = fmaxf(mx[j], x[j][i]); }
    }
    // format 1: the group is y = z / s (s > 0); format 2 codes z = Xr / r itself (s folded
    // into the stored scale and zero)
    const float to_g = FMT == 1 ? is_own : 1.f;
    // NG = 2: a group is the 64 channels of the lanes with the same bit 3 (cb < 8, cb >= 8)
    const float lo = row16_scatter8<1, NG == 1>(mn, l) * to_g;
    const float hi_ = row16_scatter8<2, NG == 1>(mx, l) * to_g;
    const int hh = NG == 1 ? 0 : (l >> 3) & 1;
    const uint16_t sc16 = meta16((hi_ - lo) * (BITS == 2 ? 1.f / 3.f : 1.f / 15.f));
    const uint16_t zr16 = meta16(lo);
    const float sc = h2f(sc16);
    const float inv = sc > 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;
    if (NG == 2 || (l & 8) == 0) {
      sm.meta[slot_scale<FMT, NG>(hh)][tok(tok_own)] = sc16;
      sm.meta[slot_zero<FMT, NG>(hh)][tok(tok_own)] = zr16;
    }
    float* ga = &sm.gc[w][r][hh][0][0];
    float* gb = &sm.gc[w][r][hh][1][0];
    ga[tok_own] = to_g * inv;
    gb[tok_own] = -h2f(zr16) * inv;
    float A[8], B[8];
    lds_read8(ga, A);
    lds_read8(gb, B);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo4 = 0, hi4 = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = fminf(fmaf(x[j][i], A[j], B[j]), BITS == 2 ? 3.f : 15.f);
        if (j < 4) lo4 = __builtin_amdgcn_cvt_pk_u8_f32(u, j, lo4);
        else hi4 = __builtin_amdgcn_cvt_pk_u8_f32(u, j - 4, hi4);
      }
      // slots 0..3 and 4..7 are two runs of 4 consecutive tokens
      sm.codes[codes_row(8 * cb + i) + tok(0) / 4] = lo4;
      sm.codes[codes_row(8 * cb + i) + tok(4) / 4] = hi4;
    }
  }
  __syncthreads();

  // ---- 4c. value codes into the record layout; metadata ---------------------------------
  if constexpr (KIND == 1 && BITS == 4) {
    // 2048 words: word (c, g, m); nibble q = v + 4 e <- token 32m + (j < 4 ? 4g + j : 12 + 4g + j),
    // j = 2v + e (the 2-bit records' token order, one nibble per code)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int wi = tid + kThreads * k;
      const int c = wi >> 4, g = (wi >> 2) & 3, m = wi & 3;
      const uint32_t* row = &sm.codes[codes_row(c)];
      const uint32_t a = row[8 * m + g];       // slots 0..3
      const uint32_t b = row[8 * m + 4 + g];   // slots 4..7
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t code = (j < 4 ? a >> (8 * j) : b >> (8 * (j - 4))) & 15u;
        word |= code << (4 * ((j >> 1) + 4 * (j & 1)));
      }
      out[wi] = word;
    }
  } else if constexpr (KIND == 1) {
    // 1024 words: word (c, g, d); crumb p <- token 32s + (j < 4 ? 4g + j : 12 + 4g + j),
    // i = p % 8, s = 2d + i / 4, j = 2 (i % 4) + p / 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int wi = tid + kThreads * k;
      const int c = wi >> 3, g = (wi >> 1) & 3, d = wi & 1;
      const uint32_t* row = &sm.codes[codes_row(c)];
      uint32_t word = 0;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {  // the two 32-token steps of this word
        const int s_ = 2 * d + sl;
        const uint32_t a = row[8 * s_ + g];       // slots 0..3
        const uint32_t b = row[8 * s_ + 4 + g];   // slots 4..7
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // slot 2v -> low-half crumb i = 4 sl + v, slot 2v+1 -> high-half crumb 8 + i
          const int s0 = 2 * v, s1 = 2 * v + 1;
          const uint32_t c0 = s0 < 4 ? (a >> (8 * s0)) & 3 : (b >> (8 * (s0 - 4))) & 3;
          const uint32_t c1 = s1 < 4 ? (a >> (8 * s1)) & 3 : (b >> (8 * (s1 - 4))) & 3;
          const int i = 4 * sl + v;
          word |= c0 << (2 * i);
          word |= c1 << (2 * (8 + i));
        }
      }
      out[wi] = word;
    }
  }
  // metadata: meta_slots x 128 float16 (3 to 6 slots: 192 to 384 words)
  {
    const int codes_words = RecFormat<KIND, BITS, FMT, NG>::kCodeBytes / 4;
    const uint16_t* mm = &sm.meta[0][0];
#pragma unroll
    for (int k = tid; k < meta_bytes<FMT, NG>() / 4; k += kThreads)
      out[codes_words + k] = uint32_t(mm[2 * k]) | (uint32_t(mm[2 * k + 1]) << 16);
  }
}

// Four workgroups per CU (16 waves) keep a whole layer's tiles resident in one round.
template <int KIND, int BITS, int FMT, int NG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
quantize_tiles_kernel(const __half* __restrict__ src, int64_t token_stride, int64_t head_stride,
                      int64_t src_num_tokens, const int64_t* __restrict__ tile_src_token,
                      const int32_t* __restrict__ tile_dst_page, int32_t num_kv_heads,
                      uint8_t* __restrict__ pool, int64_t pool_num_pages, int n_iters) {
  __shared__ QuantSmem sm;
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = tile_src_token[tile];
  const int64_t page = tile_dst_page[tile];
  if (t0 < 0 || t0 > src_num_tokens - kTile || page < 0 || page >= pool_num_pages) return;
  const __half* base = src + t0 * token_stride + int64_t(h) * head_stride;
  auto row_ptr = [=](int t) { return base + int64_t(t) * token_stride; };
  constexpr int kRec = RecFormat<KIND, BITS, FMT, NG>::kRecord;
  uint8_t* rec = pool + (page * num_kv_heads + h) * int64_t(kRec);
  quantize_tile<KIND, BITS, FMT, NG>(row_ptr, rec, n_iters, sm);
}

// Keys and values of the same tiles in one launch: grid (n_tiles, num_kv_heads, 2), z = kind.
template <int KB, int VB, int FMT, int NG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
quantize_kv_kernel(const __half* __restrict__ k_src, const __half* __restrict__ v_src,
                   int64_t token_stride, int64_t head_stride, int64_t src_num_tokens,
                   const int64_t* __restrict__ tile_src_token,
                   const int32_t* __restrict__ tile_dst_page, int32_t num_kv_heads,
                   uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                   int64_t pool_num_pages, int n_iters) {
  __shared__ QuantSmem sm;
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_k = blockIdx.z == 0;
  const int64_t t0 = tile_src_token[tile];
  const int64_t page = tile_dst_page[tile];
  if (t0 < 0 || t0 > src_num_tokens - kTile || page < 0 || page >= pool_num_pages) return;
  const __half* base = (is_k ? k_src : v_src) + t0 * token_stride + int64_t(h) * head_stride;
  auto row_ptr = [=](int t) { return base + int64_t(t) * token_stride; };
  if (is_k)
    quantize_tile<0, KB, FMT, NG>(row_ptr, k_pool + (page * num_kv_heads + h) * int64_t(RecFormat<0, KB, FMT, NG>::kRecord),
                         n_iters, sm);
  else
    quantize_tile<1, VB, FMT, NG>(row_ptr, v_pool + (page * num_kv_heads + h) * int64_t(RecFormat<1, VB, FMT, NG>::kRecord),
                         n_iters, sm);
}

// Append one token per (sequence, head) into staging; quantize the staging tile it fills.
// grid: (batch, num_kv_heads, 2 kinds)
template <int KB, int VB, int FMT, int NG>
__global__ void __launch_bounds__(kThreads)
append_tokens_kernel(const __half* __restrict__ k_new, const __half* __restrict__ v_new,
                     int32_t num_kv_heads, const int32_t* __restrict__ seq_lens,
                     __half* __restrict__ k_tail, __half* __restrict__ v_tail,
                     const int32_t* __restrict__ block_table, int32_t bt_stride,
                     uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                     int64_t pool_num_pages, int n_iters) {
  __shared__ QuantSmem sm;
  const int b = blockIdx.x, h = blockIdx.y, kind = blockIdx.z;
  const int32_t L = seq_lens[b];
  if (L < 0) return;
  const int slot = L % kTile;
  const __half* src_new = (kind == 0 ? k_new : v_new) + (int64_t(b) * num_kv_heads + h) * kDim;
  __half* stage = (kind == 0 ? k_tail : v_tail) + (int64_t(b) * num_kv_heads + h) * kTile * kDim;
  const int tid = threadIdx.x;
  if (tid < 16) {
    *reinterpret_cast<uint4*>(stage + slot * kDim + 8 * tid) =
        *reinterpret_cast<const uint4*>(src_new + 8 * tid);
  }
  if (slot != kTile - 1 || L / kTile >= bt_stride) return;
  const int64_t page = block_table[int64_t(b) * bt_stride + L / kTile];
  if (page < 0 || page >= pool_num_pages) return;
  // the filled row is read from the new-token buffer, never from the staging just written
  auto row_ptr = [=](int t) { return t == kTile - 1 ? src_new : stage + int64_t(t) * kDim; };
  if (kind == 0) {
    quantize_tile<0, KB, FMT, NG>(row_ptr, k_pool + (page * num_kv_heads + h) * int64_t(RecFormat<0, KB, FMT, NG>::kRecord),
                         n_iters, sm);
  } else {
    quantize_tile<1, VB, FMT, NG>(row_ptr, v_pool + (page * num_kv_heads + h) * int64_t(RecFormat<1, VB, FMT, NG>::kRecord),
                         n_iters, sm);
  }
}

// Chunk write, part 1: every tile that the chunk completes is quantized into its page.
// Sequence b holds L = seq_lens[b] tokens before the chunk and receives n tokens, rows
// cu_new[b] .. cu_new[b] + n - 1 of the token-major new-token buffers, at positions L .. L+n-1.
// grid: (tile slots, batch, num_kv_heads * 2); slot j is tile t = L / 128 + j, quantized when
// complete (128 t + 128 <= L + n). Its rows below L come from staging (only the tile that was
// partial before the chunk has such rows), the others straight from the new-token buffer.
template <int KB, int VB, int FMT, int NG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
write_tiles_kernel(const __half* __restrict__ k_new, const __half* __restrict__ v_new,
                   int32_t total_new, const int32_t* __restrict__ cu_new, int32_t max_new,
                   int32_t num_kv_heads,
                   const int32_t* __restrict__ seq_lens, const __half* __restrict__ k_tail,
                   const __half* __restrict__ v_tail, const int32_t* __restrict__ block_table,
                   int32_t bt_stride, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                   int64_t pool_num_pages, int n_iters) {
  __shared__ QuantSmem sm;
  const int b = blockIdx.y;
  const int h = blockIdx.z >> 1, kind = blockIdx.z & 1;
  const int32_t L = seq_lens[b];
  const int32_t c0 = cu_new[b];
  int32_t n = cu_new[b + 1] - c0;
  n = n < 0 ? 0 : (n > max_new ? max_new : n);
  if (L < 0 || c0 < 0 || int64_t(c0) + n > total_new) return;   // rows outside the buffers
  const int64_t t = int64_t(L / kTile) + blockIdx.x;
  const int64_t end = int64_t(L) + n;
  if (t * kTile + kTile > end || t >= bt_stride) return;     // not completed by this chunk
  const int64_t page = block_table[int64_t(b) * bt_stride + t];
  if (page < 0 || page >= pool_num_pages) return;
  const int64_t row_stride = int64_t(num_kv_heads) * kDim;
  const __half* src = (kind == 0 ? k_new : v_new) + int64_t(c0) * row_stride + int64_t(h) * kDim;
  const __half* stage = (kind == 0 ? k_tail : v_tail) + (int64_t(b) * num_kv_heads + h) * kTile * kDim;
  const int64_t t0 = t * kTile;
  auto row_ptr = [=](int r) {
    const int64_t a = t0 + r;
    return a < L ? stage + int64_t(r) * kDim : src + (a - L) * row_stride;
  };
  if (kind == 0)
    quantize_tile<0, KB, FMT, NG>(row_ptr, k_pool + (page * num_kv_heads + h) * int64_t(RecFormat<0, KB, FMT, NG>::kRecord),
                         n_iters, sm);
  else
    quantize_tile<1, VB, FMT, NG>(row_ptr, v_pool + (page * num_kv_heads + h) * int64_t(RecFormat<1, VB, FMT, NG>::kRecord),
                         n_iters, sm);
}

// Chunk write, part 2 (after part 1, which reads the staging rows this overwrites): the new
// tokens of the partial last tile, positions max(L, 128 floor((L+n)/128)) .. L+n-1, go to
// staging rows position mod 128. grid: (batch, num_kv_heads, 2 kinds); 16 bytes per thread.
__global__ void __launch_bounds__(kThreads)
write_staging_kernel(const __half* __restrict__ k_new, const __half* __restrict__ v_new,
                     int32_t total_new, const int32_t* __restrict__ cu_new, int32_t max_new,
                     int32_t num_kv_heads,
                     const int32_t* __restrict__ seq_lens, __half* __restrict__ k_tail,
                     __half* __restrict__ v_tail) {
  const int b = blockIdx.x, h = blockIdx.y, kind = blockIdx.z;
  const int32_t L = seq_lens[b];
  const int32_t c0 = cu_new[b];
  int32_t n = cu_new[b + 1] - c0;
  n = n < 0 ? 0 : (n > max_new ? max_new : n);
  if (L < 0 || n == 0 || c0 < 0 || int64_t(c0) + n > total_new) return;
  const int64_t end = int64_t(L) + n;
  const int64_t first = end / kTile * kTile > L ? end / kTile * kTile : L;   // first staged position
  const int rows = int(end - first);                                          // 0 .. 127
  const int64_t row_stride = int64_t(num_kv_heads) * kDim;
  const __half* src = (kind == 0 ? k_new : v_new) + int64_t(c0) * row_stride + int64_t(h) * kDim;
  __half* stage = (kind == 0 ? k_tail : v_tail) + (int64_t(b) * num_kv_heads + h) * kTile * kDim;
  for (int i = threadIdx.x; i < rows * 16; i += kThreads) {
    const int r = i >> 4, c = (i & 15) * 8;
    const int64_t a = first + r;
    *reinterpret_cast<uint4*>(stage + (a % kTile) * kDim + c) =
        *reinterpret_cast<const uint4*>(src + (a - L) * row_stride + c);
  }
}

// Page records back to float16 tiles (read side, then the inverse rotation H^-1 = H):
// grid (n_tiles, num_kv_heads), one workgroup per record, the thread layout of the
// quantizer (channels 8cb..+7 x tokens 8tb..+7). dst: [n_tiles][num_kv_heads][token][channel].
template <int KIND, int BITS, int FMT, int NG>
__global__ void __launch_bounds__(kThreads)
dequantize_tiles_kernel(const uint8_t* __restrict__ pool, int64_t pool_num_pages,
                        const int32_t* __restrict__ pages, int32_t num_kv_heads,
                        __half* __restrict__ dst) {
  constexpr int kRec = RecFormat<KIND, BITS, FMT, NG>::kRecord;
  // metadata slots: format 1 r, s, scales, zeros; format 2 keys s, scales', zeros' (r = 1),
  // values r, scales', zeros' (s = 1); NG = 2: the scale and zero of half h (token / 64 for
  // keys, channel / 64 for values) in slots slot_scale(h), slot_zero(h)
  constexpr int kR = 0, kS = FMT == 1 ? 1 : 0;
  constexpr bool kHasR = FMT == 1 || KIND == 1, kHasS = FMT == 1 || KIND == 0;
  __shared__ uint4 rec_sm[(kRec + 15) / 16];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int64_t page = pages[tile];
  if (page < 0 || page >= pool_num_pages) return;
  const uint4* rec = reinterpret_cast<const uint4*>(pool + (page * num_kv_heads + h) * int64_t(kRec));
  const int tid = threadIdx.x;
  for (int i = tid; i < kRec / 16; i += kThreads) rec_sm[i] = rec[i];   // kRec % 16 == 0
  __syncthreads();
  const uint32_t* words = reinterpret_cast<const uint32_t*>(rec_sm);
  const uint16_t* meta = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const uint8_t*>(rec_sm) + RecFormat<KIND, BITS, FMT, NG>::kCodeBytes);
  const int w = tid >> 6, l = tid & 63, cb = l & 15, tb = 4 * w + (l >> 4);
  float x[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = 8 * tb + j;
    const float st = kHasS ? h2f(meta[kS * kTile + t]) : 1.f;
    uint32_t kw = 0;
    if constexpr (KIND == 0 && BITS == 4) kw = words[t * 16 + cb];   // channels 8cb..8cb+7 of token t
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * cb + i;
      uint32_t code;
      float sc, zr;
      if constexpr (KIND == 0) {
        if constexpr (BITS == 4) {
          code = (kw >> (4 * ((i & 1) ? 4 + (i >> 1) : (i >> 1)))) & 15u;   // nibble of channel i
        } else {   // word c / 16 of token t, crumb 4 hs + v + 8 e, hs = bit 3 of c
          const int hs = (c >> 3) & 1;
          const int p = 4 * hs + ((c & 7) >> 1) + 8 * (c & 1);
          code = (words[t * 8 + (c >> 4)] >> (2 * p)) & 3u;
        }
        const int hg = NG == 1 ? 0 : t >> 6;
        sc = h2f(meta[slot_scale<FMT, NG>(hg) * kDim + c]);
        zr = h2f(meta[slot_zero<FMT, NG>(hg) * kDim + c]);
      } else {
        // token t of channel c: word 8c + 2g + d, crumb p (the record's crumb order)
        const int s_ = t >> 5, rem = t & 31;
        const int g = rem < 16 ? rem >> 2 : (rem - 16) >> 2;
        const int jj = rem < 16 ? rem & 3 : 4 + (rem & 3);
        if constexpr (BITS == 2) {
          const int p = 4 * (s_ & 1) + (jj >> 1) + 8 * (jj & 1);
          code = (words[8 * c + 2 * g + (s_ >> 1)] >> (2 * p)) & 3u;
        } else {   // word (c, g, m = s_), nibble (jj / 2) + 4 (jj % 2)
          const int qn = (jj >> 1) + 4 * (jj & 1);
          code = (words[16 * c + 4 * g + s_] >> (4 * qn)) & 15u;
        }
        const int hg = NG == 1 ? 0 : c >> 6;
        sc = h2f(meta[slot_scale<FMT, NG>(hg) * kDim + t]);
        zr = h2f(meta[slot_zero<FMT, NG>(hg) * kDim + t]);
      }
      x[j][i] = (kHasR ? h2f(meta[kR * kDim + c]) : 1.f) * st * fmaf(sc, float(code), zr);
    }
  }
  fwht_channels_f32(x, cb);
  __half* out = dst + (int64_t(tile) * num_kv_heads + h) * kTile * kDim;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint4 v;
    v.x = uint32_t(f2h_rn(x[j][0])) | (uint32_t(f2h_rn(x[j][1])) << 16);
    v.y = uint32_t(f2h_rn(x[j][2])) | (uint32_t(f2h_rn(x[j][3])) << 16);
    v.z = uint32_t(f2h_rn(x[j][4])) | (uint32_t(f2h_rn(x[j][5])) << 16);
    v.w = uint32_t(f2h_rn(x[j][6])) | (uint32_t(f2h_rn(x[j][7])) << 16);
    *reinterpret_cast<uint4*>(out + (8 * tb + j) * kDim + 8 * cb) = v;
  }
}

}  // namespace

hipError_t launch_dequantize_tiles(int kind, int k_bits, int v_bits, int fmt, int group, const void* pool,
                                   int64_t pool_num_pages, const int32_t* pages, int32_t n_tiles,
                                   int32_t num_kv_heads, void* dst, hipStream_t stream) {
  dim3 grid(n_tiles, num_kv_heads), block(kThreads);
  const auto* pl = static_cast<const uint8_t*>(pool);
  auto* d = static_cast<__half*>(dst);
  return with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    if (kind == 1)
      hipLaunchKernelGGL((dequantize_tiles_kernel<1, decltype(vb)::value, decltype(fm)::value, decltype(ng)::value>), grid, block, 0, stream,
                         pl, pool_num_pages, pages, num_kv_heads, d);
    else
      hipLaunchKernelGGL((dequantize_tiles_kernel<0, decltype(kb)::value, decltype(fm)::value, decltype(ng)::value>), grid, block, 0, stream,
                         pl, pool_num_pages, pages, num_kv_heads, d);
  });
}

hipError_t launch_quantize_tiles(int kind, int k_bits, int v_bits, int fmt, int group, const void* src,
                                 int64_t token_stride, int64_t head_stride, int64_t src_num_tokens,
                                 const int64_t* tile_src_token, const int32_t* tile_dst_page,
                                 int32_t n_tiles, int32_t num_kv_heads, void* pool,
                                 int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  dim3 grid(n_tiles, num_kv_heads), block(kThreads);
  const auto* sp = static_cast<const __half*>(src);
  auto* pl = static_cast<uint8_t*>(pool);
  return with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    if (kind == 1)
      hipLaunchKernelGGL((quantize_tiles_kernel<1, decltype(vb)::value, decltype(fm)::value, decltype(ng)::value>), grid, block, 0, stream,
                         sp, token_stride, head_stride, src_num_tokens, tile_src_token,
                         tile_dst_page, num_kv_heads, pl, pool_num_pages, n_iters);
    else
      hipLaunchKernelGGL((quantize_tiles_kernel<0, decltype(kb)::value, decltype(fm)::value, decltype(ng)::value>), grid, block, 0, stream,
                         sp, token_stride, head_stride, src_num_tokens, tile_src_token,
                         tile_dst_page, num_kv_heads, pl, pool_num_pages, n_iters);
  });
}

hipError_t launch_quantize_kv(int k_bits, int v_bits, int fmt, int group, const void* k_src, const void* v_src,
                              int64_t token_stride, int64_t head_stride, int64_t src_num_tokens,
                              const int64_t* tile_src_token, const int32_t* tile_dst_page,
                              int32_t n_tiles, int32_t num_kv_heads, void* k_pool, void* v_pool,
                              int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  dim3 grid(n_tiles, num_kv_heads, 2), block(kThreads);
  const auto* ks = static_cast<const __half*>(k_src);
  const auto* vs = static_cast<const __half*>(v_src);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  return with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    hipLaunchKernelGGL((quantize_kv_kernel<decltype(kb)::value, decltype(vb)::value, decltype(fm)::value, decltype(ng)::value>), grid, block,
                       0, stream, ks, vs, token_stride, head_stride, src_num_tokens,
                       tile_src_token, tile_dst_page, num_kv_heads, kp, vp, pool_num_pages,
                       n_iters);
  });
}

hipError_t launch_write_tokens(int k_bits, int v_bits, int fmt, int group, const void* k_new, const void* v_new,
                               int32_t total_new, const int32_t* cu_new, int32_t max_new,
                               int32_t batch, int32_t num_kv_heads, const int32_t* seq_lens,
                               void* k_tail, void* v_tail, const int32_t* block_table,
                               int32_t bt_stride, void* k_pool, void* v_pool,
                               int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  // tiles completed by n tokens: at most n / 128 + 1
  dim3 grid1(max_new / kTile + 1, batch, num_kv_heads * 2), block(kThreads);
  const auto* kn = static_cast<const __half*>(k_new);
  const auto* vn = static_cast<const __half*>(v_new);
  const hipError_t e = with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    hipLaunchKernelGGL((write_tiles_kernel<decltype(kb)::value, decltype(vb)::value, decltype(fm)::value, decltype(ng)::value>), grid1,
                       block, 0, stream, kn, vn, total_new, cu_new, max_new, num_kv_heads,
                       seq_lens, static_cast<const __half*>(k_tail),
                       static_cast<const __half*>(v_tail), block_table, bt_stride,
                       static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                       pool_num_pages, n_iters);
  });
  if (e != hipSuccess) return e;
  dim3 grid2(batch, num_kv_heads, 2);
  hipLaunchKernelGGL(write_staging_kernel, grid2, block, 0, stream, kn, vn, total_new, cu_new,
                     max_new, num_kv_heads, seq_lens, static_cast<__half*>(k_tail),
                     static_cast<__half*>(v_tail));
  return hipGetLastError();
}

hipError_t launch_append_tokens(int k_bits, int v_bits, int fmt, int group, const void* k_new, const void* v_new,
                                int32_t batch, int32_t num_kv_heads, const int32_t* seq_lens,
                                void* k_tail, void* v_tail, const int32_t* block_table,
                                int32_t bt_stride, void* k_pool, void* v_pool,
                                int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  dim3 grid(batch, num_kv_heads, 2), block(kThreads);
  const auto* kn = static_cast<const __half*>(k_new);
  const auto* vn = static_cast<const __half*>(v_new);
  auto* kt = static_cast<__half*>(k_tail);
  auto* vt = static_cast<__half*>(v_tail);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  return with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    hipLaunchKernelGGL((append_tokens_kernel<decltype(kb)::value, decltype(vb)::value, decltype(fm)::value, decltype(ng)::value>), grid,
                       block, 0, stream, kn, vn, num_kv_heads, seq_lens, kt, vt, block_table,
                       bt_stride, kp, vp, pool_num_pages, n_iters);
  });
}

}  // namespace kvarn

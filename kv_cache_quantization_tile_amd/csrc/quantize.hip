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
// Thread layout: thread (wave w, lane l) owns the 8x8 block channels 8cb..8cb+7 x tokens
// 8tb..8tb+7 with cb = l % 16 and tb = 4w + l / 16. Reductions over channels stay inside a
// 16-lane row (DPP); reductions over tokens combine the 4 rows of a wave (swizzle /
// bpermute) and the 4 waves through LDS. The tile stays in registers (64 fp32 / thread).
#include "kvarn_device.h"
#include "kvarn_launch.h"

// Sums and products below are written in the order the numerics need; no contraction.
#pragma clang fp contract(off)

namespace kvarn {
namespace {

constexpr int kThreads = 256;

struct QuantSmem {
  float red[2][4][16][8];      // per-wave partials of token-direction reductions (2 buffers)
  uint8_t codes[kTile * kDim]; // K: [token][channel]; V: [channel][token]
  uint16_t meta[4][kDim];      // r, s, scale, zero as float16 bits
};

// Sum (or min / max) of 8 per-thread values over the 16 token blocks of the tile; every
// thread receives the totals for its own 8 channels. op: 0 sum, 1 min, 2 max. `buf`
// alternates between calls so one barrier per call suffices (a buffer is rewritten only
// after the other buffer's barrier).
template <int OP>
__device__ __forceinline__ void reduce_over_tokens(float (&v)[8], QuantSmem& sm, int w, int l, int buf) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = swz_xor_f<16>(v[i]);
    if constexpr (OP == 0) v[i] += o;
    else if constexpr (OP == 1) v[i] = fminf(v[i], o);
    else v[i] = fmaxf(v[i], o);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = shfl_xor32_f(v[i]);
    if constexpr (OP == 0) v[i] += o;
    else if constexpr (OP == 1) v[i] = fminf(v[i], o);
    else v[i] = fmaxf(v[i], o);
  }
  const int cb = l & 15;
  if (l < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.red[buf][w][cb][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = sm.red[buf][0][cb][i], b = sm.red[buf][1][cb][i];
    const float c = sm.red[buf][2][cb][i], d = sm.red[buf][3][cb][i];
    if constexpr (OP == 0) v[i] = (a + b) + (c + d);
    else if constexpr (OP == 1) v[i] = fminf(fminf(a, b), fminf(c, d));
    else v[i] = fmaxf(fmaxf(a, b), fmaxf(c, d));
  }
}

// Sum of each of 8 values over the 16 lanes of a row, all values stage by stage so the DPP
// reads never wait on the instruction just before them.
__device__ __forceinline__ void row16_sum8(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_f<kDppQuadXor1>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_f<kDppQuadXor2>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_f<kDppHalfMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_f<kDppRowRor8>(v[i]);
}

// FWHT of length 128 along channels for each of the thread's 8 tokens, then * 1/sqrt(128).
// Channel bits 0..2 are in-thread; bits 3..6 are lane bits 0..3. A cross-lane butterfly
// stage on lane bit m is one fused multiply-add per value: y += c * y(lane ^ m) with c = +1
// on lanes whose bit m is 0 and -1 on the others. Lanes with the bit set then hold the
// negated difference; the accumulated sign, (-1)^popcount(lane bits 0..3), is removed by the
// final scaling.
__device__ __forceinline__ void fwht_channels(float (&x)[8][8], int cb) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
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
  // partners of one token's 8 values are fetched before any of them is updated
#define KVARN_XSTAGE(FETCH, C)                                              \
  _Pragma("unroll") for (int j = 0; j < 8; ++j) {                           \
    float p[8];                                                             \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) p[i] = FETCH(x[j][i]);    \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) x[j][i] = fmaf(p[i], C, x[j][i]); \
  }
  KVARN_XSTAGE(dpp_f<kDppQuadXor1>, c1)
  KVARN_XSTAGE(dpp_f<kDppQuadXor2>, c2)
  KVARN_XSTAGE(swz_xor_f<4>, c4)
  KVARN_XSTAGE(dpp_f<kDppRowRor8>, c8)
#undef KVARN_XSTAGE
  const float fin = (__builtin_popcount(cb) & 1) ? -kInvSqrt128 : kInvSqrt128;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[j][i] *= fin;
}

// The tile quantizer proper. row_ptr(t) gives the 16-byte aligned address of token t's
// 128 channels. Writes one record at `rec`.
template <int KIND, typename RowPtr>
__device__ void quantize_tile(RowPtr row_ptr, uint8_t* __restrict__ rec, int n_iters, QuantSmem& sm) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int cb = l & 15;
  const int tb = 4 * w + (l >> 4);

  // ---- 1. gather: token 8tb+j, channels 8cb..8cb+7 (16 bytes) --------------------------
  float x[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row_ptr(8 * tb + j) + 8 * cb);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[j][2 * k] = h2f(uint16_t(wds[k] & 0xFFFF));
      x[j][2 * k + 1] = h2f(uint16_t(wds[k] >> 16));
    }
  }

  // ---- 2. rotate --------------------------------------------------------------------
  fwht_channels(x, cb);

  // ---- 3. normalize -----------------------------------------------------------------
  // Two passes per step (mean, then centred sum of squares), float32 FMAs. The next step's
  // weights are 1/std = rsqrt(var). A group whose variance is below 1e-12 mean^2 is constant
  // up to float32 rounding (a non-constant group of float16-derived values has a relative
  // spread of at least ~1e-5): its update is skipped, as for an exactly zero std.
  float ir[8], is[8];      // 1/r for my channels, 1/s for my tokens
  float vr[8], vs[8];      // last accepted variances (r = sqrt(vr), s = sqrt(vs)); 1 = never
#pragma unroll
  for (int i = 0; i < 8; ++i) { ir[i] = 1.f; is[i] = 1.f; vr[i] = 1.f; vs[i] = 1.f; }
  int buf = 0;
  for (int it = 0; it < n_iters; ++it) {
    // column step: per token, over the 128 channels (8 in-thread x 16 lanes of the row)
    float m[8], q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaf(x[j][i], ir[i], a);
      m[j] = a;
    }
    row16_sum8(m);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m[j] *= -(1.f / kDim);                 // minus the mean
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = fmaf(x[j][i], ir[i], m[j]);
        a = fmaf(d, d, a);
      }
      q[j] = a;
    }
    row16_sum8(q);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float var = q[j] * (1.f / kDim);
      vs[j] = var > 1e-12f * m[j] * m[j] ? var : vs[j];
      is[j] = __builtin_amdgcn_rsqf(vs[j]);
    }
    // row step: per channel, over the 128 tokens (8 in-thread x 16 token blocks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaf(x[j][i], is[j], a);
      m[i] = a;
    }
    reduce_over_tokens<0>(m, sm, w, l, buf);
    buf ^= 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m[i] *= -(1.f / kTile);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = fmaf(x[j][i], is[j], m[i]);
        a = fmaf(d, d, a);
      }
      q[i] = a;
    }
    reduce_over_tokens<0>(q, sm, w, l, buf);
    buf ^= 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float var = q[i] * (1.f / kTile);
      vr[i] = var > 1e-12f * m[i] * m[i] ? var : vr[i];
      ir[i] = __builtin_amdgcn_rsqf(vr[i]);
    }
  }
  float r[8], s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r[i] = __builtin_amdgcn_sqrtf(vr[i]);
    s[i] = __builtin_amdgcn_sqrtf(vs[i]);
  }

  // ---- 4a. stored normalizers and the normalized tile --------------------------------
  uint16_t r16[8], s16[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r16[i] = f2h_rn(fminf(fmaxf(r[i], 6.103515625e-05f), 65504.f));
    ir[i] = __builtin_amdgcn_rcpf(h2f(r16[i]));
    s16[i] = f2h_rn(fminf(fmaxf(s[i], 6.103515625e-05f), 65504.f));
    is[i] = __builtin_amdgcn_rcpf(h2f(s16[i]));
  }
  // lanes of wave 0, row 0 hold every channel's r; the lanes of column 0 every token's s
  if (tb == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.meta[0][8 * cb + i] = r16[i];
  }
  if (cb == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.meta[1][8 * tb + j] = s16[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[j][i] = (x[j][i] * is[j]) * ir[i];

  // ---- 4b. asymmetric RTN -----------------------------------------------------------
  if constexpr (KIND == 0) {
    // keys: one group per channel, over the 128 tokens
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn[i] = x[0][i];
      mx[i] = x[0][i];
#pragma unroll
      for (int j = 1; j < 8; ++j) { mn[i] = fminf(mn[i], x[j][i]); mx[i] = fmaxf(mx[i], x[j][i]); }
    }
    reduce_over_tokens<1>(mn, sm, w, l, 0);
    reduce_over_tokens<2>(mx, sm, w, l, 1);
    uint16_t sc16[8], zr16[8];
    float inv[8], off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sc16[i] = f2h_rn((mx[i] - mn[i]) * (1.f / 15.f));
      zr16[i] = f2h_rn(mn[i]);
      const float sc = h2f(sc16[i]);
      inv[i] = sc > 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;
      off[i] = -h2f(zr16[i]) * inv[i];
    }
    if (tb == 0) {  // every channel's group statistics
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sm.meta[2][8 * cb + i] = sc16[i];
        sm.meta[3][8 * cb + i] = zr16[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // code = clamp(rne((y - zero) / scale), 0, 15), packed one byte per code
        const float u = __builtin_amdgcn_fmed3f(__builtin_rintf(fmaf(x[j][i], inv[i], off[i])), 0.f, 15.f);
        if (i < 4) lo = __builtin_amdgcn_cvt_pk_u8_f32(u, i, lo);
        else hi = __builtin_amdgcn_cvt_pk_u8_f32(u, i - 4, hi);
      }
      *reinterpret_cast<uint2*>(&sm.codes[(8 * tb + j) * kDim + 8 * cb]) = make_uint2(lo, hi);
    }
  } else {
    // values: one group per token, over the 128 channels
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = x[j][0], b = x[j][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) { a = fminf(a, x[j][i]); b = fmaxf(b, x[j][i]); }
      mn[j] = row16_min(a);
      mx[j] = row16_max(b);
    }
    uint16_t sc16[8], zr16[8];
    float inv[8], off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sc16[j] = f2h_rn((mx[j] - mn[j]) * (1.f / 3.f));
      zr16[j] = f2h_rn(mn[j]);
      const float sc = h2f(sc16[j]);
      inv[j] = sc > 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;
      off[j] = -h2f(zr16[j]) * inv[j];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = __builtin_amdgcn_fmed3f(__builtin_rintf(fmaf(x[j][i], inv[j], off[j])), 0.f, 3.f);
        if (j < 4) lo = __builtin_amdgcn_cvt_pk_u8_f32(u, j, lo);
        else hi = __builtin_amdgcn_cvt_pk_u8_f32(u, j - 4, hi);
      }
      *reinterpret_cast<uint2*>(&sm.codes[(8 * cb + i) * kTile + 8 * tb]) = make_uint2(lo, hi);
    }
    if (cb == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sm.meta[2][8 * tb + j] = sc16[j];
        sm.meta[3][8 * tb + j] = zr16[j];
      }
    }
  }
  __syncthreads();

  // ---- 4c. pack codes into the record layout and store -------------------------------
  uint32_t* out = reinterpret_cast<uint32_t*>(rec);
  if constexpr (KIND == 0) {
    // 2048 words: word (t, j) = channels 8j..8j+7 of token t, nibble p <- channel
    // 8j + {0,2,4,6,1,3,5,7}[p]
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int wi = tid + kThreads * k;
      const int t = wi >> 4, j = wi & 15;
      const uint2 c8 = *reinterpret_cast<const uint2*>(&sm.codes[t * kDim + 8 * j]);
      // byte q of c8 = code of channel 8j+q; even channels to nibbles 0..3, odd to 4..7
      const uint32_t e = (c8.x & 0xFF) | ((c8.x >> 8) & 0xFF00) | ((c8.y & 0xFF) << 16) | ((c8.y & 0xFF0000) << 8);
      const uint32_t o = ((c8.x >> 8) & 0xFF) | ((c8.x >> 16) & 0xFF00) | (((c8.y >> 8) & 0xFF) << 16) | ((c8.y >> 24) << 24);
      // e, o hold 4 codes as bytes; compress bytes to nibbles
      const uint32_t en = (e & 0xF) | ((e >> 4) & 0xF0) | ((e >> 8) & 0xF00) | ((e >> 12) & 0xF000);
      const uint32_t on = (o & 0xF) | ((o >> 4) & 0xF0) | ((o >> 8) & 0xF00) | ((o >> 12) & 0xF000);
      out[wi] = en | (on << 16);
    }
  } else {
    // 1024 words: word (c, g, d); crumb p <- token 32s + (j < 4 ? 4g + j : 12 + 4g + j),
    // i = p % 8, s = 2d + i / 4, j = 2 (i % 4) + p / 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int wi = tid + kThreads * k;
      const int c = wi >> 3, g = (wi >> 1) & 3, d = wi & 1;
      const uint8_t* row = &sm.codes[c * kTile];
      uint32_t word = 0;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {  // the two 32-token steps of this word
        const int s = 2 * d + sl;
        const uint32_t a = *reinterpret_cast<const uint32_t*>(row + 32 * s + 4 * g);       // slots 0..3
        const uint32_t b = *reinterpret_cast<const uint32_t*>(row + 32 * s + 16 + 4 * g);  // slots 4..7
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
  // metadata: 4 x 128 float16 = 256 words, one per thread
  {
    const int codes_words = (KIND == 0 ? kKCodeBytes : kVCodeBytes) / 4;
    const uint16_t* m = &sm.meta[0][0];
    out[codes_words + tid] = uint32_t(m[2 * tid]) | (uint32_t(m[2 * tid + 1]) << 16);
  }
}

// Four workgroups per CU (16 waves) keep a whole layer's tiles resident in one round.
template <int KIND>
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
  constexpr int kRec = KIND == 0 ? kKRecord : kVRecord;
  uint8_t* rec = pool + (page * num_kv_heads + h) * int64_t(kRec);
  quantize_tile<KIND>(row_ptr, rec, n_iters, sm);
}

// Keys and values of the same tiles in one launch: grid (n_tiles, num_kv_heads, 2), z = kind.
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
    quantize_tile<0>(row_ptr, k_pool + (page * num_kv_heads + h) * int64_t(kKRecord), n_iters, sm);
  else
    quantize_tile<1>(row_ptr, v_pool + (page * num_kv_heads + h) * int64_t(kVRecord), n_iters, sm);
}

// Append one token per (sequence, head) into staging; quantize the staging tile it fills.
// grid: (batch, num_kv_heads, 2 kinds)
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
    quantize_tile<0>(row_ptr, k_pool + (page * num_kv_heads + h) * int64_t(kKRecord), n_iters, sm);
  } else {
    quantize_tile<1>(row_ptr, v_pool + (page * num_kv_heads + h) * int64_t(kVRecord), n_iters, sm);
  }
}

}  // namespace

hipError_t launch_quantize_tiles(int kind, const void* src, int64_t token_stride,
                                 int64_t head_stride, int64_t src_num_tokens,
                                 const int64_t* tile_src_token, const int32_t* tile_dst_page,
                                 int32_t n_tiles, int32_t num_kv_heads, void* pool,
                                 int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  dim3 grid(n_tiles, num_kv_heads), block(kThreads);
  if (kind == 0) {
    hipLaunchKernelGGL(quantize_tiles_kernel<0>, grid, block, 0, stream,
                       static_cast<const __half*>(src), token_stride, head_stride, src_num_tokens,
                       tile_src_token, tile_dst_page, num_kv_heads, static_cast<uint8_t*>(pool),
                       pool_num_pages, n_iters);
  } else {
    hipLaunchKernelGGL(quantize_tiles_kernel<1>, grid, block, 0, stream,
                       static_cast<const __half*>(src), token_stride, head_stride, src_num_tokens,
                       tile_src_token, tile_dst_page, num_kv_heads, static_cast<uint8_t*>(pool),
                       pool_num_pages, n_iters);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const void* k_src, const void* v_src, int64_t token_stride,
                              int64_t head_stride, int64_t src_num_tokens,
                              const int64_t* tile_src_token, const int32_t* tile_dst_page,
                              int32_t n_tiles, int32_t num_kv_heads, void* k_pool, void* v_pool,
                              int64_t pool_num_pages, int n_iters, hipStream_t stream) {
  dim3 grid(n_tiles, num_kv_heads, 2), block(kThreads);
  hipLaunchKernelGGL(quantize_kv_kernel, grid, block, 0, stream,
                     static_cast<const __half*>(k_src), static_cast<const __half*>(v_src),
                     token_stride, head_stride, src_num_tokens, tile_src_token, tile_dst_page,
                     num_kv_heads, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                     pool_num_pages, n_iters);
  return hipGetLastError();
}

hipError_t launch_append_tokens(const void* k_new, const void* v_new, int32_t batch,
                                int32_t num_kv_heads, const int32_t* seq_lens, void* k_tail,
                                void* v_tail, const int32_t* block_table, int32_t bt_stride,
                                void* k_pool, void* v_pool, int64_t pool_num_pages, int n_iters,
                                hipStream_t stream) {
  dim3 grid(batch, num_kv_heads, 2), block(kThreads);
  hipLaunchKernelGGL(append_tokens_kernel, grid, block, 0, stream,
                     static_cast<const __half*>(k_new), static_cast<const __half*>(v_new),
                     num_kv_heads, seq_lens, static_cast<__half*>(k_tail),
                     static_cast<__half*>(v_tail), block_table, bt_stride,
                     static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                     pool_num_pages, n_iters);
  return hipGetLastError();
}

}  // namespace kvarn

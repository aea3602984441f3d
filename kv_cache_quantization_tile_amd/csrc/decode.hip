// KVarN paged decode attention for gfx950: split-K over 128-token pages, MFMA on the
// quantized codes, online softmax, float16 tail, log-sum-exp merge and H^T.
//
// Algebra (KVarN README, "How KVarN works": the rotation is orthonormal so scores are
// preserved, and the scales are re-applied on read -- keys per channel, values per token).
// A key page stores Xr = H K^T as r_c s_t (zero_c + scale_c code_ct). With q_rot = H q:
//   q . k_t = s_t ( sum_c q''_c code_ct + q_rot . (r * zero) ),   q'' = q_rot * r * scale.
// A value page stores r_c s_t (zero_t + scale_t code_ct), so for weights p_t
//   sum_t p_t (H^T-rotated v_t) = r * ( sum_t (p_t s_t scale_t) code_t + sum_t p_t s_t zero_t )
// and the output is H^T acc / l after the splits are merged.
//
// MFMA v_mfma_f32_16x16x32_f16, lane l: A row l%16, k 8(l/16)..+7; B column l%16, same k;
// C rows 4(l/16)..+3, column l%16.
//   QK: A = key codes (rows = 16 tokens, k = 32 channels), B = q'' (columns: 8 heads as
//       float16 high parts, then the same 8 heads' low parts), C = scores.
//   PV: A = value codes (rows = 16 channels, k = 32 tokens), B = p s scale (high / low),
//       C = partial outputs. The k-order of the tokens in a PV step is the order in which
//       the QK C-fragments hold them, which is the value record's crumb order.
// Codes enter the MFMA as normal float16 numbers 1 + code/16 (keys: the nibble is moved into
// mantissa bits 6..9 under the exponent of 1.0) and 1 + code/4 (values: the crumb into bits
// 8..9). The MFMA then returns sum_k B_k + sum_k B_k code_k / 16 (or / 4); the kernel subtracts
// the column sum of its own B operand, a cancellation of about 3x. Subnormal operands are
// avoided on purpose: the matrix core accumulates products of subnormal inputs with visibly
// less than float32 precision.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPartStride = 132;  // floats per partial: m, l, pad, pad, acc[128]
constexpr int kMaxMergeSplits = 4096;  // splits one merge workgroup can weight (LDS)

__device__ __forceinline__ float4v mfma16x16x32(const half8& a, const half8& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

union H8 {
  half8 v;
  uint32_t u[4];
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return uint32_t(f2h_rn(a)) | (uint32_t(f2h_rn(b)) << 16);
}

// float16 high part (hi == true) or float16 low part f16(x - f32(f16(x))) of a float, returned
// as the exact float value of that float16
__device__ __forceinline__ float split16(float x, bool hi) {
  const float h = h2f(f2h_rn(x));
  return hi ? h : h2f(f2h_rn(x - h));
}

// (t & mask) | magic in one 3-input bit operation (truth table 0xEA: S0 & S1 | S2)
__device__ __forceinline__ uint32_t and_or(uint32_t t, uint32_t mask, uint32_t magic) {
  return __builtin_amdgcn_bitop3_b32(t, mask, magic, 0xEA);
}

// key codes of word w, nibble pair v (nibbles v and 4 + v), as float16x2 1 + code / 16
__device__ __forceinline__ uint32_t k_pair(uint32_t w, int v) {
  const uint32_t t = v == 0 ? (w << 6) : v == 1 ? (w << 2) : v == 2 ? (w >> 2) : (w >> 6);
  return and_or(t, 0x03C003C0u, 0x3C003C00u);
}

// value codes of word w, crumb pair i (crumbs i and 8 + i), as float16x2 1 + code / 4
__device__ __forceinline__ uint32_t v_pair(uint32_t w, int i) {
  const int sh = 8 - 2 * i;
  const uint32_t t = sh >= 0 ? (w << sh) : (w >> -sh);
  return and_or(t, 0x03000300u, 0x3C003C00u);
}

// 2^x on the transcendental unit (results below 2^-126 flush to 0, which softmax weights
// of that size may)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void load_h4(const uint8_t* p, float (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = h2f(uint16_t(v.x & 0xFFFF));
  o[1] = h2f(uint16_t(v.x >> 16));
  o[2] = h2f(uint16_t(v.y & 0xFFFF));
  o[3] = h2f(uint16_t(v.y >> 16));
}

__device__ __forceinline__ void load_h8(const uint8_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = h2f(uint16_t(w[k] & 0xFFFF));
    o[2 * k + 1] = h2f(uint16_t(w[k] >> 16));
  }
}

struct DecodeSmem {
  float m[4][8];
  float l[4][8];
  float acc[4][8][kDim];
};

// One workgroup: (split, KV head g, sequence b). Wave w handles page slots
// split * 4 * tpw + w + 4 k, k < tpw. Writes one partial (m, l, acc) per query head.
__global__ void __launch_bounds__(kThreads)
decode_pages_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                    int64_t pool_num_pages, const int32_t* __restrict__ block_table,
                    int32_t bt_stride, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    float qscale, int32_t tpw, int32_t n_splits, float* __restrict__ ws) {
  __shared__ DecodeSmem sm;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = num_q_heads / num_kv_heads;
  int32_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  const int n_full = L / kTile;
  const int slot0 = split * 4 * tpw;
  if (slot0 >= n_full) return;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n = l & 15, gq = l >> 4;
  const int h = n & 7;
  const bool hi = n < 8;
  const bool head_ok = h < G;

  // ---- q_rot = H q * softmax_scale * log2(e): lane holds channels 32 gq + j ----------
  float qr[32];
  {
    const __half* qrow = q + (int64_t(b) * num_q_heads + int64_t(g) * G + (head_ok ? h : 0)) * kDim + 32 * gq;
#pragma unroll
    for (int k = 0; k < 4; ++k) load_h8(reinterpret_cast<const uint8_t*>(qrow + 8 * k), &qr[8 * k]);
    if (!head_ok) {
#pragma unroll
      for (int j = 0; j < 32; ++j) qr[j] = 0.f;
    }
#pragma unroll
    for (int hb = 1; hb < 32; hb <<= 1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if ((j & hb) == 0) {
          const float a = qr[j], c = qr[j + hb];
          qr[j] = a + c;
          qr[j + hb] = a - c;
        }
      }
    }
    const bool up16 = (gq & 1) != 0, up32 = (gq & 2) != 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = swz_xor_f<16>(qr[j]);
      qr[j] = up16 ? (p - qr[j]) : (qr[j] + p);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = shfl_xor32_f(qr[j]);
      qr[j] = up32 ? (p - qr[j]) : (qr[j] + p);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) qr[j] *= qscale;  // includes 1/sqrt(128) of H
  }

  float m_run = -INFINITY, l_run = 0.f;
  float acc[8][4];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[bb][i] = 0.f;

  for (int k = 0; k < tpw; ++k) {
    const int slot = slot0 + w + 4 * k;
    if (slot >= n_full) break;
    const int64_t page = block_table[int64_t(b) * bt_stride + slot];
    if (page < 0 || page >= pool_num_pages) continue;
    const uint8_t* krec = k_pool + (page * num_kv_heads + g) * int64_t(kKRecord);
    const uint8_t* vrec = v_pool + (page * num_kv_heads + g) * int64_t(kVRecord);

    // ---- B operand of QK: q'' for my 32 channels; bias q_rot . (r * zero) ------------
    H8 bq[4];
    float bias, bsum;
    {
      float bpart = 0.f, bs = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // channels 32 gq + 8 s + (0..7) = k-step s
        float rr[8], sc8[8], zr8[8];
        load_h8(krec + kKCodeBytes + 0 * 256 + (32 * gq + 8 * s) * 2, rr);
        load_h8(krec + kKCodeBytes + 2 * 256 + (32 * gq + 8 * s) * 2, sc8);
        load_h8(krec + kKCodeBytes + 3 * 256 + (32 * gq + 8 * s) * 2, zr8);
#pragma unroll
        for (int j = 0; j < 8; ++j) bpart = fmaf(qr[8 * s + j] * rr[j], zr8[j], bpart);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float b0 = split16(qr[8 * s + 2 * v] * rr[2 * v] * sc8[2 * v], hi);
          const float b1 = split16(qr[8 * s + 2 * v + 1] * rr[2 * v + 1] * sc8[2 * v + 1], hi);
          bs += b0 + b1;
          bq[s].u[v] = pack_h2(b0, b1);
        }
      }
      bias = rows4_sum(bpart);
      bsum = rows4_sum(bs);                     // column sum of my B operand, 128 channels
      bsum += dpp_f<kDppRowRor8>(bsum);         // high + low columns
    }
    // score = s_t * (16 (C_hi + C_lo) - 16 (sum B_hi + sum B_lo) + bias)
    const float bias16 = fmaf(-16.f, bsum, bias);

    // ---- QK ---------------------------------------------------------------------------
    float sc_[8][4];
    {
      uint4 kc[8];
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
        kc[tb] = *reinterpret_cast<const uint4*>(krec + (16 * tb + n) * 64 + 16 * gq);
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        float4v c = {0.f, 0.f, 0.f, 0.f};
        const uint32_t dw[4] = {kc[tb].x, kc[tb].y, kc[tb].z, kc[tb].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          H8 a;
#pragma unroll
          for (int v = 0; v < 4; ++v) a.u[v] = k_pair(dw[s], v);
          c = mfma16x16x32(a.v, bq[s].v, c);
        }
        float st[4];
        load_h4(krec + kKCodeBytes + 256 + (16 * tb + 4 * gq) * 2, st);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float full = c[i] + dpp_f<kDppRowRor8>(c[i]);  // high + low columns
          sc_[tb][i] = st[i] * fmaf(full, 16.f, bias16);
        }
      }
    }

    // ---- online softmax ------------------------------------------------------------------
    float mt = sc_[0][0];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc_[tb][i]);
    mt = rows4_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2_fast(m_run - m_new);
    float psum = 0.f, bz = 0.f, bsum_p = 0.f;
    H8 bp[4];
    {
      float pw[8][4];
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        float vs[4], vsc[4], vz[4];
        load_h4(vrec + kVCodeBytes + 256 + (16 * tb + 4 * gq) * 2, vs);
        load_h4(vrec + kVCodeBytes + 512 + (16 * tb + 4 * gq) * 2, vsc);
        load_h4(vrec + kVCodeBytes + 768 + (16 * tb + 4 * gq) * 2, vz);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_fast(sc_[tb][i] - m_new);
          psum += p;
          const float ps = p * vs[i];
          bz = fmaf(ps, vz[i], bz);
          pw[tb][i] = split16(ps * vsc[i], hi);
          bsum_p += pw[tb][i];
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bp[s].u[0] = pack_h2(pw[2 * s][0], pw[2 * s][1]);
        bp[s].u[1] = pack_h2(pw[2 * s][2], pw[2 * s][3]);
        bp[s].u[2] = pack_h2(pw[2 * s + 1][0], pw[2 * s + 1][1]);
        bp[s].u[3] = pack_h2(pw[2 * s + 1][2], pw[2 * s + 1][3]);
      }
    }
    psum = rows4_sum(psum);
    bz = rows4_sum(bz);
    // the MFMA returns sum_t B_t (1 + code_t / 4); remove the 1s, add the zero-point term
    const float corr = fmaf(-4.f, rows4_sum(bsum_p), hi ? bz : 0.f);
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;

    // ---- PV ---------------------------------------------------------------------------
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const uint2 vc = *reinterpret_cast<const uint2*>(vrec + (16 * bb + n) * 32 + 8 * gq);
      float4v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t word = d ? vc.y : vc.x;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          H8 a;
#pragma unroll
          for (int v = 0; v < 4; ++v) a.u[v] = v_pair(word, 4 * hs + v);
          c = mfma16x16x32(a.v, bp[2 * d + hs].v, c);
        }
      }
      float rv[4];
      load_h4(vrec + kVCodeBytes + (16 * bb + 4 * gq) * 2, rv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = fmaf(c[i], 4.f, corr);
        acc[bb][i] = fmaf(acc[bb][i], alpha, rv[i] * o);
      }
    }
  }

  // ---- combine the high / low columns, then the 4 waves --------------------------------
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[bb][i] += dpp_f<kDppRowRor8>(acc[bb][i]);
  if (hi) {
    if (gq == 0) {
      sm.m[w][h] = m_run;
      sm.l[w][h] = l_run;
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[w][h][16 * bb + 4 * gq + i] = acc[bb][i];
  }
  __syncthreads();
  {
    const int hh = tid >> 5;           // head 0..7
    const int c0 = (tid & 31) * 4;     // 4 channels
    if (hh < G) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm.m[ww][hh]);
      float e[4], Lt = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        e[ww] = (M == -INFINITY) ? 0.f : exp2f(sm.m[ww][hh] - M);
        Lt = fmaf(e[ww], sm.l[ww][hh], Lt);
      }
      float* part = ws + ((int64_t(b) * num_q_heads + int64_t(g) * G + hh) * (n_splits + 1) + split) * kPartStride;
      float4 o;
      float* op = &o.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) a = fmaf(e[ww], sm.acc[ww][hh][c0 + i], a);
        op[i] = a;
      }
      *reinterpret_cast<float4*>(part + 4 + c0) = o;
      if ((tid & 31) == 0) {
        part[0] = M;
        part[1] = Lt;
      }
    }
  }
}

// Exact attention over the float16 tail (tokens past the last full page), raw space.
// One workgroup per (KV head g, sequence b); wave w handles heads 2w, 2w+1 of the group.
__global__ void __launch_bounds__(kThreads)
decode_tail_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                   const __half* __restrict__ k_tail, const __half* __restrict__ v_tail,
                   const int32_t* __restrict__ seq_lens, int32_t max_seq_len, float qscale,
                   int32_t n_splits, float* __restrict__ ws) {
  __shared__ float p_sm[8][kTile];
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = num_q_heads / num_kv_heads;
  int32_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  const int T = L % kTile;
  if (T == 0) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const __half* kt = k_tail + (int64_t(b) * num_kv_heads + g) * kTile * kDim;
  const __half* vt = v_tail + (int64_t(b) * num_kv_heads + g) * kTile * kDim;
  for (int hh = 2 * w; hh < 2 * w + 2; ++hh) {
    if (hh >= G) break;
    const int hq = g * G + hh;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q + (int64_t(b) * num_q_heads + hq) * kDim);
    float sc[2];
#pragma unroll
    for (int half_ = 0; half_ < 2; ++half_) {
      const int t = l + 64 * half_;
      float a = -INFINITY;
      if (t < T) {
        a = 0.f;
        const uint8_t* krow = reinterpret_cast<const uint8_t*>(kt + int64_t(t) * kDim);
        for (int c8 = 0; c8 < 16; ++c8) {
          float qv[8], kv[8];
          load_h8(qrow + 16 * c8, qv);
          load_h8(krow + 16 * c8, kv);
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qv[i], kv[i], a);
        }
        a *= qscale;
      }
      sc[half_] = a;
    }
    float mx = fmaxf(sc[0], sc[1]);
    for (int off = 1; off < 64; off <<= 1)
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(((l ^ off) << 2), __float_as_int(mx))));
    float ps = 0.f;
#pragma unroll
    for (int half_ = 0; half_ < 2; ++half_) {
      const int t = l + 64 * half_;
      const float p = t < T ? exp2f(sc[half_] - mx) : 0.f;
      p_sm[hh][t] = p;
      ps += p;
    }
    for (int off = 1; off < 64; off <<= 1)
      ps += __int_as_float(__builtin_amdgcn_ds_bpermute(((l ^ off) << 2), __float_as_int(ps)));
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    float o0 = 0.f, o1 = 0.f;
    for (int t = 0; t < T; ++t) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(vt + int64_t(t) * kDim + 2 * l);
      const float p = p_sm[hh][t];
      o0 = fmaf(p, h2f(uint16_t(vv & 0xFFFF)), o0);
      o1 = fmaf(p, h2f(uint16_t(vv >> 16)), o1);
    }
    float* part = ws + ((int64_t(b) * num_q_heads + hq) * (n_splits + 1) + n_splits) * kPartStride;
    *reinterpret_cast<float2*>(part + 4 + 2 * l) = make_float2(o0, o1);
    if (l == 0) {
      part[0] = mx;
      part[1] = ps;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Merge the splits of one (sequence, query head): log-sum-exp weights, H^T on the page
// part (rotated space), plus the raw-space tail; float16 output. One 128-thread workgroup
// per (query head, sequence): thread c owns channel c; split weights are computed once in
// LDS, then every thread streams its channel of all partials (independent loads).
__global__ void __launch_bounds__(128)
decode_merge_kernel(int32_t num_q_heads, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    int32_t tiles_per_split, int32_t n_splits, int32_t has_tail,
                    const float* __restrict__ ws, __half* __restrict__ out) {
  __shared__ float wsh[kMaxMergeSplits + 1];
  __shared__ float red[2][2];
  __shared__ float xs[kDim];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int c = threadIdx.x, lane = c & 63, wv = c >> 6;
  int32_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  const int n_full = L / kTile;
  const int used = (n_full + tiles_per_split - 1) / tiles_per_split;
  const bool tail = has_tail && (L % kTile) != 0;
  const float* base = ws + (int64_t(b) * num_q_heads + hq) * (n_splits + 1) * kPartStride;
  // 1. global max over the used splits (and the tail)
  float M = -INFINITY;
  for (int s = c; s < used; s += 128) M = fmaxf(M, base[s * kPartStride]);
  if (tail && c == 0) M = fmaxf(M, base[n_splits * kPartStride]);
  for (int off = 32; off >= 1; off >>= 1)
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(M))));
  if (lane == 0) red[0][wv] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  // 2. split weights exp2(m_s - M) and the total l
  float lsum = 0.f;
  for (int s = c; s < used; s += 128) {
    const float e = M == -INFINITY ? 0.f : exp2f(base[s * kPartStride] - M);
    wsh[s] = e;
    lsum = fmaf(e, base[s * kPartStride + 1], lsum);
  }
  if (c == 0) {
    const float e = (tail && M != -INFINITY) ? exp2f(base[n_splits * kPartStride] - M) : 0.f;
    wsh[kMaxMergeSplits] = e;
    if (tail) lsum = fmaf(e, base[n_splits * kPartStride + 1], lsum);
  }
  for (int off = 32; off >= 1; off >>= 1)
    lsum += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(lsum)));
  if (lane == 0) red[1][wv] = lsum;
  __syncthreads();
  lsum = red[1][0] + red[1][1];
  // 3. weighted sum of the rotated accumulators, channel c
  float a = 0.f;
  int s = 0;
  for (; s + 4 <= used; s += 4) {
    const float v0 = base[(s + 0) * kPartStride + 4 + c];
    const float v1 = base[(s + 1) * kPartStride + 4 + c];
    const float v2 = base[(s + 2) * kPartStride + 4 + c];
    const float v3 = base[(s + 3) * kPartStride + 4 + c];
    a = fmaf(wsh[s], v0, a);
    a = fmaf(wsh[s + 1], v1, a);
    a = fmaf(wsh[s + 2], v2, a);
    a = fmaf(wsh[s + 3], v3, a);
  }
  for (; s < used; ++s) a = fmaf(wsh[s], base[s * kPartStride + 4 + c], a);
  // 4. H^T = H over the 128 channels: bits 0..5 across the lanes of a wave, bit 6 via LDS
  {
#define KVARN_MSTAGE(M_, FN)                          \
    {                                                 \
      const float p = FN(a);                          \
      a = (lane & (M_)) ? (p - a) : (a + p);          \
    }
    KVARN_MSTAGE(1, dpp_f<kDppQuadXor1>)
    KVARN_MSTAGE(2, dpp_f<kDppQuadXor2>)
    KVARN_MSTAGE(4, swz_xor_f<4>)
    KVARN_MSTAGE(8, dpp_f<kDppRowRor8>)
    KVARN_MSTAGE(16, swz_xor_f<16>)
    KVARN_MSTAGE(32, shfl_xor32_f)
#undef KVARN_MSTAGE
    xs[c] = a;
    __syncthreads();
    const float p = xs[c ^ 64];
    a = (c & 64) ? (p - a) : (a + p);
    a *= kInvSqrt128;
  }
  if (tail) a = fmaf(wsh[kMaxMergeSplits], base[n_splits * kPartStride + 4 + c], a);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  out[(int64_t(b) * num_q_heads + hq) * kDim + c] = __float2half_rn(a * inv);
}

}  // namespace

int32_t decode_tiles_per_wave(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t max_full = max_seq_len / kTile;
  const int64_t work = int64_t(batch) * num_kv_heads * max_full;
  int64_t tpw = (work + 4095) / 4096;       // aim at ~4096 page-waves of work per wave slot
  if (tpw < 1) tpw = 1;
  if (tpw > 64) tpw = 64;
  // the merge weighs at most kMaxMergeSplits splits of 4 * tpw pages each
  const int64_t need = (max_full + 4LL * kMaxMergeSplits - 1) / (4LL * kMaxMergeSplits);
  if (tpw < need) tpw = need;
  return int32_t(tpw);
}

int32_t decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int32_t tpw = decode_tiles_per_wave(batch, num_kv_heads, max_seq_len);
  const int32_t max_full = max_seq_len / kTile;
  int32_t ns = (max_full + 4 * tpw - 1) / (4 * tpw);
  return ns < 1 ? 1 : ns;
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_seq_len) {
  const int32_t ns = decode_num_splits(batch, num_kv_heads, max_seq_len);
  return size_t(batch) * num_q_heads * (ns + 1) * kPartStride * sizeof(float);
}

hipError_t launch_decode(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         const void* k_pool, const void* v_pool, int64_t pool_num_pages,
                         const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                         int32_t max_seq_len, const void* k_tail, const void* v_tail,
                         float softmax_scale, void* workspace, void* out, hipStream_t stream) {
  const int32_t tpw = decode_tiles_per_wave(batch, num_kv_heads, max_seq_len);
  const int32_t ns = decode_num_splits(batch, num_kv_heads, max_seq_len);
  const float qscale = softmax_scale * kLog2e;
  float* ws = static_cast<float*>(workspace);
  if (max_seq_len >= kTile) {
    hipLaunchKernelGGL(decode_pages_kernel, dim3(ns, num_kv_heads, batch), dim3(kThreads), 0, stream,
                       static_cast<const __half*>(q), num_q_heads, num_kv_heads,
                       static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool),
                       pool_num_pages, block_table, bt_stride, seq_lens, max_seq_len,
                       qscale * kInvSqrt128, tpw, ns, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool has_tail = k_tail != nullptr && v_tail != nullptr;
  if (has_tail) {
    hipLaunchKernelGGL(decode_tail_kernel, dim3(num_kv_heads, batch), dim3(kThreads), 0, stream,
                       static_cast<const __half*>(q), num_q_heads, num_kv_heads,
                       static_cast<const __half*>(k_tail), static_cast<const __half*>(v_tail),
                       seq_lens, max_seq_len, qscale, ns, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_merge_kernel, dim3(num_q_heads, batch), dim3(128), 0, stream,
                     num_q_heads, seq_lens, max_seq_len, 4 * tpw, ns, has_tail ? 1 : 0,
                     static_cast<const float*>(ws), static_cast<__half*>(out));
  return hipGetLastError();
}

}  // namespace kvarn

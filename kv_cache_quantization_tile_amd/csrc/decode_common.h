// Device helpers shared by the decode and multi-query read kernels (decode.hip, mq.hip):
// page record geometry and loads, code unpacking into float16 MFMA operands, per-page
// factors, the geometry of an output row, and the exact attention over a staged tail.
// Internal to the library; each including source gets its own copies.
#pragma once

#include "kvarn_device.h"

namespace kvarn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPartStride = 132;  // floats per partial: m, l, pad, pad, acc[128]
constexpr int kMaxMergeSplits = 4000;  // splits one merge wave can weight (4 heads x (4000 + 1) floats of LDS < 64 KB)
// Balanced decode layout (one query row per sequence): at most this many sequences (their
// page prefix sums live in LDS) and 4 * kBalancedPageWg page waves (one round of 2 waves per
// SIMD on 256 CUs).
constexpr int kMaxBalancedRows = 1024;
constexpr int kBalancedPageWg = 512;

// Floats of the balanced layout's page partials: one slot per (page wave, segment) index sum
// i + (b Hkv + g), G query heads each; the tail partials (one per (row, query head)) follow.
__host__ __device__ inline int64_t balanced_tail_offset(int32_t n_page_wg, int32_t batch,
                                                        int32_t num_q_heads,
                                                        int32_t num_kv_heads) {
  return (4 * int64_t(n_page_wg) + int64_t(batch) * num_kv_heads) *
         (num_q_heads / num_kv_heads) * kPartStride;
}
// ... and the page prefix sums (batch + 1 int32: full pages before each sequence, then the
// total) after the tail partials.
__host__ __device__ inline int64_t balanced_pref_offset(int32_t n_page_wg, int32_t batch,
                                                        int32_t num_q_heads,
                                                        int32_t num_kv_heads) {
  return balanced_tail_offset(n_page_wg, batch, num_q_heads, num_kv_heads) +
         int64_t(batch) * num_q_heads * kPartStride;
}

__device__ __forceinline__ float4v mfma16x16x32(const half8& a, const half8& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

union H8 {
  half8 v;
  uint32_t u[4];
};

// (t & mask) | magic in one 3-input bit operation (truth table 0xEA: S0 & S1 | S2)
__device__ __forceinline__ uint32_t and_or(uint32_t t, uint32_t mask, uint32_t magic) {
  return __builtin_amdgcn_bitop3_b32(t, mask, magic, 0xEA);
}

// Key codes of word w, nibble pair v (nibbles v and 4 + v = channels 2v and 2v + 1 of the
// word's 8), as float16x2 1 + code * 2^(b - 10): the nibbles go to mantissa bits b..b+3 with
// b = 2 for even v and b = 6 for odd v, so two shifted copies of the word serve all four pairs.
// The operand on the other side carries the matching factor 2^(10 - b) (256 or 16).
__device__ __forceinline__ uint32_t k_pair(uint32_t w, int v) {
  const uint32_t t = v < 2 ? (w << 2) : (w >> 6);
  return and_or(t, (v & 1) ? 0x03C003C0u : 0x003C003Cu, 0x3C003C00u);
}

// Value codes of word w, crumb pair i (crumbs i and 8 + i), as float16x2 1 + code * 2^(b - 10):
// b = 8 for even i, 6 for odd i (factor 4 or 16 on the other side); four shifted copies.
__device__ __forceinline__ uint32_t v_pair(uint32_t w, int i) {
  const int sh = i == 0 ? 8 : i <= 2 ? 4 : i <= 4 ? 0 : i <= 6 ? -4 : -8;
  const uint32_t t = sh >= 0 ? (w << sh) : (w >> -sh);
  return and_or(t, (i & 1) ? 0x00C000C0u : 0x03000300u, 0x3C003C00u);
}

// 2^x on the transcendental unit (results below 2^-126 flush to 0, which softmax weights
// of that size may)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void load_h8(const uint8_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = h2f(uint16_t(w[k] & 0xFFFF));
    o[2 * k + 1] = h2f(uint16_t(w[k] >> 16));
  }
}

// Per wave: the float32 factors of the page being processed.
//   ka[c] = r_c scale_c 2^(10-b_c) ks      kb[c] = ks r_c zero_c - ka[c]     kt[t] = s_t / ks
//   vp[t] = s_t scale_t 2^(10-b_t) vs      vz[t] = vs s_t zero_t - vp[t]     vr[c] = r_c / vs
// (ks, vs: the page's powers of two for the B operands.) With NG = 2 (group 64) the key
// factors ka, kb come per token half (tokens 64 h ..) and the value factors vp, vz per
// channel half (channels 64 h ..).
template <int NG>
struct WaveMeta {
  float4 ka[NG][kDim / 4], kb[NG][kDim / 4];   // read 4 channels at a time
  float2 kt[kTile / 2], vp[NG][kTile / 2], vz[NG][kTile / 2];   // read 2 tokens at a time
  float4 vr[kDim / 4];
};


// Raw loads of one page: key codes (16 B per 16-token block at 4 bits, 8 B at 2), value
// codes (8 B per 16-channel block at 2 bits, 16 B at 4), and entries 2l, 2l+1 of each
// float16 metadata array of the records.
// Key record geometry by key code width (4: kvarn_k4v2_g128 / kvarn_k4v4_g128,
// 2: kvarn_k2v2_g128).
template <int KB> struct KeyRec;
template <> struct KeyRec<4> {
  static constexpr int kRecord = kKRecord, kCodeBytes = kKCodeBytes;
  typedef uint4 Codes;    // one 16-token block: 4 words = the 4 k-steps of 8 channels
};
template <> struct KeyRec<2> {
  static constexpr int kRecord = kK2Record, kCodeBytes = kK2CodeBytes;
  typedef uint2 Codes;    // one 16-token block: 2 words, each 2 k-steps of 8 channels
};

// Value record geometry by value code width (2: kvarn_k4v2_g128 / kvarn_k2v2_g128,
// 4: kvarn_k4v4_g128).
template <int VB> struct ValRec;
template <> struct ValRec<2> {
  static constexpr int kRecord = kVRecord, kCodeBytes = kVCodeBytes;
  typedef uint2 Codes;    // one 16-channel block: 2 words, each 2 k-steps of 8 tokens
};
template <> struct ValRec<4> {
  static constexpr int kRecord = kV4Record, kCodeBytes = kV4CodeBytes;
  typedef uint4 Codes;    // one 16-channel block: 4 words = the 4 k-steps of 8 tokens
};

// Record bytes by code width and format.
template <int KB, int FMT, int NG> constexpr int key_record() { return KeyRec<KB>::kCodeBytes + meta_bytes<FMT, NG>(); }
template <int VB, int FMT, int NG> constexpr int val_record() { return ValRec<VB>::kCodeBytes + meta_bytes<FMT, NG>(); }

template <int KB, int VB>
struct PageRegs {
  typename KeyRec<KB>::Codes kc[8];
  typename ValRec<VB>::Codes vc[8];
  uint32_t km[kMaxMetaSlots], vm[kMaxMetaSlots];   // the first meta_slots are loaded
};

// Page loads through buffer descriptors: one scalar descriptor per record (base, size), a
// 32-bit per-lane offset fixed for the kernel and a scalar offset per load, so no per-load
// address arithmetic runs on the vector ALU (and reads past the record return 0).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;   // raw (untyped) 32-bit data
// Page records are read once per decode step: nontemporal loads (cache policy bit nt) keep
// them from displacing reused lines (measured: 0.85 vs 0.75 of HBM peak for this pattern).
// In a multi-query read the waves of one workgroup (other rows of the same sequence) stream
// the same pages at about the same time: there the loads are plain (kReuseLoad), so that
// the others find the page in L2.
constexpr int kStreamLoad = 2;
constexpr int kReuseLoad = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec), (short)0, bytes, kBufferFlags);
}

struct LaneOffsets {
  uint32_t k, v, m;   // key codes, value codes, metadata
};

template <int AUX, int FMT, int NG, int KB, int VB>
__device__ __forceinline__ void load_meta(PageRegs<KB, VB>& t, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, const LaneOffsets& o) {
#pragma unroll
  for (int a = 0; a < meta_slots<FMT, NG>(); ++a) {
    t.km[a] = __builtin_amdgcn_raw_buffer_load_b32(kr, o.m, KeyRec<KB>::kCodeBytes + 256 * a, AUX);
    t.vm[a] = __builtin_amdgcn_raw_buffer_load_b32(vr, o.m, ValRec<VB>::kCodeBytes + 256 * a, AUX);
  }
}
template <int AUX, int KB, int VB>
__device__ __forceinline__ void load_kcodes(PageRegs<KB, VB>& t, __amdgpu_buffer_rsrc_t kr,
                                            const LaneOffsets& o) {
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) {
    if constexpr (KB == 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(kr, o.k, 1024 * tb, AUX);
      t.kc[tb] = make_uint4(v.x, v.y, v.z, v.w);
    } else {   // 32 bytes per token: the value records' lane offsets
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(kr, o.v, 512 * tb, AUX);
      t.kc[tb] = make_uint2(v.x, v.y);
    }
  }
}
template <int AUX, int KB, int VB>
__device__ __forceinline__ void load_vcodes(PageRegs<KB, VB>& t, __amdgpu_buffer_rsrc_t vr,
                                            const LaneOffsets& o) {
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    if constexpr (VB == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(vr, o.v, 512 * bb, AUX);
      t.vc[bb] = make_uint2(v.x, v.y);
    } else {   // 64 bytes per channel: the 4-bit key records' lane offsets
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(vr, o.k, 1024 * bb, AUX);
      t.vc[bb] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
}

__device__ __forceinline__ float lo_h(uint32_t w) { return h2f(uint16_t(w & 0xFFFF)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f(uint16_t(w >> 16)); }

__device__ __forceinline__ float wave_max(float v) { return rows4_max(row16_max(v)); }

// Exponent k = 14 - e for x = m 2^e, m in [0.5, 1): x 2^k lies in [2^13, 2^14). 0 when x is
// zero or not finite; clamped to +-100.
__device__ __forceinline__ int pow2_norm_exp(float x) {
  if (!(x > 0.f) || !(x <= 3.4e38f)) return 0;
  const int k = 14 - __builtin_amdgcn_frexp_expf(x);
  return k < -100 ? -100 : (k > 100 ? 100 : k);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// float16x2 high parts of (a, b) and low parts f16(a - f16(a)), f16(b - f16(b)): one packed
// conversion and two mixed-precision FMAs that read the float16 high parts back in place
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  uint32_t h, r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(h) : "v"(a), "v"(b));
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(a), "v"(h));
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(r) : "v"(b), "v"(h));
  hi = h;
  lo = r;
}

// Per-lane choice between two values by an all-ones / all-zero mask (one 3-input bit
// operation, truth table 0xCA: S0 ? S1 : S2 bitwise)
__device__ __forceinline__ float pick(uint32_t mask, float if_set, float if_clear) {
  return __uint_as_float(__builtin_amdgcn_bitop3_b32(mask, __float_as_uint(if_set),
                                                     __float_as_uint(if_clear), 0xCA));
}

// DPP row_ror:8 move that only writes the lanes of the given banks (bank k = lanes 4k..4k+3
// of each 16-lane row); the other lanes keep `old`.
template <int BANKS>
__device__ __forceinline__ uint32_t swap8_into(uint32_t old, uint32_t src) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(src), kDppRowRor8, 0xF, BANKS, false));
}
constexpr int kHiBanks = 0x3;   // lanes 0..7 of a row: high-part columns
constexpr int kLoBanks = 0xC;   // lanes 8..15: low-part columns

// Page factors of the record pair held in t, for the B operands, into this wave's LDS slot
// (lane l: channels and tokens 2l, 2l + 1). fk, fv: the lane's unpack factors 2^(10 - b);
// maxq: the wave's largest |q_rot| (sets the power of two ks that keeps the QK B operand
// below 2^14; vs does the same for the PV one; both over every group of the page).
// Format 1 slots: keys and values r, s, scales, zeros. Format 2 (folded): keys s, scales',
// zeros' (r folded into the per-channel scales and zeros: rk = 1); values r, scales', zeros'
// (s folded into the per-token scales and zeros: sv = 1). NG = 2: one scale and one zero
// slot per half.
template <int FMT, int NG, int KB, int VB>
__device__ __forceinline__ void page_factors(const PageRegs<KB, VB>& t, WaveMeta<NG>& wm, int l,
                                             float maxq, float fk, float fv) {
  constexpr int kS = FMT == 1 ? 1 : 0;
  const float rk0 = FMT == 1 ? lo_h(t.km[0]) : 1.f, rk1 = FMT == 1 ? hi_h(t.km[0]) : 1.f;
  const float sv0 = FMT == 1 ? lo_h(t.vm[1]) : 1.f, sv1 = FMT == 1 ? hi_h(t.vm[1]) : 1.f;
  float ka0[NG], ka1[NG], vp0[NG], vp1[NG];
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    ka0[h] = rk0 * lo_h(t.km[slot_scale<FMT, NG>(h)]) * fk;
    ka1[h] = rk1 * hi_h(t.km[slot_scale<FMT, NG>(h)]) * fk;
    vp0[h] = sv0 * lo_h(t.vm[slot_scale<FMT, NG>(h)]) * fv;
    vp1[h] = sv1 * hi_h(t.vm[slot_scale<FMT, NG>(h)]) * fv;
    mk = h ? fmaxf(mk, fmaxf(ka0[h], ka1[h])) : fmaxf(ka0[h], ka1[h]);
    mv = h ? fmaxf(mv, fmaxf(vp0[h], vp1[h])) : fmaxf(vp0[h], vp1[h]);
  }
  const float mka = wave_max(mk);
  const float mvp = wave_max(mv);
  const int eks = pow2_norm_exp(maxq * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mka))));
  const int evs = pow2_norm_exp(__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mvp))));
  const float ks = __builtin_ldexpf(1.f, eks), iks = __builtin_ldexpf(1.f, -eks);
  const float vs = __builtin_ldexpf(1.f, evs), ivs = __builtin_ldexpf(1.f, -evs);
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    const float a0 = ka0[h] * ks, a1 = ka1[h] * ks;
    const uint32_t kz = t.km[slot_zero<FMT, NG>(h)], vzr = t.vm[slot_zero<FMT, NG>(h)];
    reinterpret_cast<float2*>(wm.ka[h])[l] = make_float2(a0, a1);
    reinterpret_cast<float2*>(wm.kb[h])[l] =
        make_float2(fmaf(ks * rk0, lo_h(kz), -a0), fmaf(ks * rk1, hi_h(kz), -a1));
    const float p0 = vp0[h] * vs, p1 = vp1[h] * vs;
    wm.vp[h][l] = make_float2(p0, p1);
    wm.vz[h][l] = make_float2(fmaf(vs * sv0, lo_h(vzr), -p0), fmaf(vs * sv1, hi_h(vzr), -p1));
  }
  wm.kt[l] = make_float2(lo_h(t.km[kS]) * iks, hi_h(t.km[kS]) * iks);
  reinterpret_cast<float2*>(wm.vr)[l] = make_float2(lo_h(t.vm[0]) * ivs, hi_h(t.vm[0]) * ivs);
}

// What one output row attends to. Decode (cu_q == nullptr): row b is sequence b, attending
// to its L = seq_lens[b] tokens: the full pages, then the L mod 128 staged tokens. Several
// queries per sequence (cu_q != nullptr): rows cu_q[b] .. cu_q[b+1]-1 are the last
// n = cu_q[b+1] - cu_q[b] positions of sequence b (its cache of C = seq_lens[b] tokens ends with
// them), row cu_q[b] + i at position C - n + i attending causally to L = C - n + i + 1 tokens.
// A partial last tile of L that is a completed page (it lies below 128 floor(C / 128)) is one
// more page slot whose tokens from L mod 128 on are masked; otherwise it is the staging tile.
struct RowGeom {
  int b;          // sequence (block table and staging row)
  int n_slots;    // page slots to stream (full pages, plus one masked page)
  int mask_lim;   // tokens of the last slot that count (128: all)
  int tail_len;   // staged tokens attended (0: none)
};

__device__ __forceinline__ RowGeom row_geometry(int row, const int32_t* __restrict__ seq_lens,
                                                int32_t max_seq_len,
                                                const int32_t* __restrict__ cu_q, int32_t batch) {
  RowGeom r;
  int32_t C, L;
  if (cu_q == nullptr) {
    r.b = row;
    C = seq_lens[row];
    C = C < 0 ? 0 : (C > max_seq_len ? max_seq_len : C);
    L = C;
  } else {
    int lo = 0, hi = batch;               // the last b with cu_q[b] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_q[mid] <= row) lo = mid; else hi = mid;
    }
    r.b = lo;
    C = seq_lens[lo];
    C = C < 0 ? 0 : (C > max_seq_len ? max_seq_len : C);
    const int32_t n = cu_q[lo + 1] - cu_q[lo];
    L = C - n + (row - cu_q[lo]) + 1;
    L = L < 0 ? 0 : (L > C ? C : L);
  }
  const int n_full = L / kTile, rem = L % kTile;
  if (rem != 0 && (n_full + 1) * kTile <= C) {
    r.n_slots = n_full + 1;
    r.mask_lim = rem;
    r.tail_len = 0;
  } else {
    r.n_slots = n_full;
    r.mask_lim = kTile;
    r.tail_len = rem;
  }
  return r;
}

// Shared memory of the staged-token attention: per wave, first its value columns staged as
// float16 rows of 32 tokens (64 channels at a time), then its partial output; the per-wave
// score maxima and weight sums.
struct TailSmem {
  float o[4][8][kDim];
  float m[4][8];
  float l[4][8];
};

// The wave's staged tokens in the order the matrix cores see them. Score block mb, row rho
// (rho = 4 j + i of the result held by lane group j) is token 16 (rho / 8) + 8 mb + rho mod 8,
// so the 8 scores of lane group j are, as the 8 contraction entries 8 j .. 8 j + 7 of the value
// product, tokens 16 (j / 2) + 8 mb + 4 (j mod 2) + i (entry 4 mb + i), and lanes 0..31 hold
// tokens 0..15, lanes 32..63 tokens 16..31 of the wave's 32.
__device__ __forceinline__ int tail_token(int mb, int rho) { return 16 * (rho >> 3) + 8 * mb + (rho & 7); }

// Exact attention over the T < 128 staged float16 tokens of (sequence sb, KV head g), raw
// space, for output row `row`: one partial (score max, weight sum, weighted value sum) per
// query head of the group, written at part0 + h head_stride (h < G <= 8). Wave w takes tokens
// 32 w .. 32 w + 31 for all heads: scores on the matrix cores (tokens x channels times
// channels x heads, heads padded to 16), its own softmax, weights times values on the matrix
// cores (the weights split into a float16 high and low part, so they keep float32 accuracy),
// the values transposed through the wave's LDS rows; the four wave partials are then merged.
// Called by all 256 threads of a workgroup (T uniform); ts must not be in use elsewhere.
__device__ void tail_partial_at(const __half* __restrict__ q, int32_t num_q_heads,
                                int32_t num_kv_heads, const __half* __restrict__ k_tail,
                                const __half* __restrict__ v_tail, int row, int sb, int g, int T,
                                float qscale, float* __restrict__ part0, int64_t head_stride,
                                TailSmem& ts) {
  const int G = num_q_heads / num_kv_heads;
  if (T == 0) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n = l & 15, j = l >> 4, hl = l >> 5;
  const int tw = 32 * w;
  const int nw = (T + 31) >> 5;   // waves with tokens (uniform); the others go to the merge
  if (w < nw) {
    const __half* kt = k_tail + (int64_t(sb) * num_kv_heads + g) * kTile * kDim;
    const __half* vt = v_tail + (int64_t(sb) * num_kv_heads + g) * kTile * kDim;
    // values first (they do not wait for the scores): phase ph, lane l holds channels
    // 64 ph + 2 (l mod 32), + 1 of tokens 16 hl + u, u < 16
    uint32_t vv[2][16];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph)
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int t = tw + 16 * hl + u;
        const __half* src = vt + int64_t(t) * kDim + 64 * ph + 2 * (l & 31);
        vv[ph][u] = t < T ? *reinterpret_cast<const uint32_t*>(src) : 0u;
      }
    // ---- scores: A = keys (16 tokens x 32 channels per k-step), B = queries (32 channels x 16
    // heads; heads from G on are zero)
    const __half* qg = q + (int64_t(row) * num_q_heads + int64_t(g) * G) * kDim;
    H8 bq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 v = n < G ? *reinterpret_cast<const uint4*>(qg + n * kDim + 32 * kk + 8 * j) : z;
      bq[kk].u[0] = v.x; bq[kk].u[1] = v.y; bq[kk].u[2] = v.z; bq[kk].u[3] = v.w;
    }
    float4v sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int t = tw + tail_token(mb, n);
      H8 a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        const __half* src = kt + int64_t(t) * kDim + 32 * kk + 8 * j;
        const uint4 v = t < T ? *reinterpret_cast<const uint4*>(src) : z;
        a[kk].u[0] = v.x; a[kk].u[1] = v.y; a[kk].u[2] = v.z; a[kk].u[3] = v.w;
      }
      sacc[mb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sacc[mb] = mfma16x16x32(a[kk].v, bq[kk].v, sacc[mb]);
    }
    // ---- this wave's softmax per head n (lanes n, n + 16, n + 32, n + 48 share a head)
    auto xor_lanes = [&](float x, int m) {
      return __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ m) << 2, __float_as_int(x)));
    };
    float sc[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tw + tail_token(mb, 4 * j + i);
        sc[mb][i] = t < T ? sacc[mb][i] * qscale : -INFINITY;
        mx = fmaxf(mx, sc[mb][i]);
      }
    mx = fmaxf(mx, xor_lanes(mx, 16));
    mx = fmaxf(mx, xor_lanes(mx, 32));
    float ps = 0.f;
    H8 ahi, alo;   // weights as the A operand of the value product: entry 4 mb + i
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sc[mb][i] - mx);   // mx is finite: the wave has a token
        ps += p;
        const _Float16 hi = _Float16(p);
        ahi.v[4 * mb + i] = hi;
        alo.v[4 * mb + i] = _Float16(p - float(hi));
      }
    ps += xor_lanes(ps, 16);
    ps += xor_lanes(ps, 32);
    // ---- weights x values: per phase, the wave's 64 value channels as LDS rows of the 32
    // tokens in contraction order (row r: 4 chunks of 8 entries, chunk c stored at c ^ (r/2 mod 4))
    uint32_t* vtr = reinterpret_cast<uint32_t*>(&ts.o[w][0][0]);
    float4v oacc[8];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      // lane l: rows 2 (l mod 32) and + 1 (the low and high channel), entries 16 hl .. 16 hl + 15;
      // entry 16 hl + e' (e' = 8 j' + 4 mb + i) is token 16 hl + 8 mb + 4 j' + i = vv[ph][u]
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const int e0 = 2 * e2, e1 = 2 * e2 + 1;
        const int u0 = 8 * ((e0 >> 2) & 1) + 4 * (e0 >> 3) + (e0 & 3);
        const int u1 = 8 * ((e1 >> 2) & 1) + 4 * (e1 >> 3) + (e1 & 3);
        lo[e2] = (vv[ph][u0] & 0xFFFFu) | (vv[ph][u1] << 16);
        hi[e2] = (vv[ph][u0] >> 16) | (vv[ph][u1] & 0xFFFF0000u);
      }
      const int r0 = 2 * (l & 31);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = 2 * hl + c2;
        const int s0 = c ^ ((r0 >> 1) & 3), s1 = c ^ (((r0 + 1) >> 1) & 3);
        *reinterpret_cast<uint4*>(vtr + 16 * r0 + 4 * s0) =
            make_uint4(lo[4 * c2], lo[4 * c2 + 1], lo[4 * c2 + 2], lo[4 * c2 + 3]);
        *reinterpret_cast<uint4*>(vtr + 16 * (r0 + 1) + 4 * s1) =
            make_uint4(hi[4 * c2], hi[4 * c2 + 1], hi[4 * c2 + 2], hi[4 * c2 + 3]);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = 16 * nb + n;
        const uint4 v = *reinterpret_cast<const uint4*>(vtr + 16 * r + 4 * (j ^ ((r >> 1) & 3)));
        H8 bv;
        bv.u[0] = v.x; bv.u[1] = v.y; bv.u[2] = v.z; bv.u[3] = v.w;
        float4v acc = mfma16x16x32(ahi.v, bv.v, float4v{0.f, 0.f, 0.f, 0.f});
        oacc[4 * ph + nb] = mfma16x16x32(alo.v, bv.v, acc);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
    }
    // ---- the wave's partial: output (head 4 j + i, channel 16 nb + n) from oacc[nb][i]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * j + i;
      if (h < G) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) ts.o[w][h][16 * nb + n] = oacc[nb][i];
      }
    }
    if (j == 0 && n < G) {
      ts.m[w][n] = mx;
      ts.l[w][n] = ps;
    }
  }
  __syncthreads();
  // ---- merge of the four wave partials: thread = head tid / 32, channels 4 (tid mod 32) + 0..3
  const int h = tid >> 5, c4 = 4 * (tid & 31);
  if (h < G) {
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mw[v] = v < nw ? ts.m[v][h] : -INFINITY;
      M = fmaxf(M, mw[v]);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v >= nw) break;
      const float f = exp2f(mw[v] - M);
      const float4 x = *reinterpret_cast<const float4*>(&ts.o[v][h][c4]);
      acc.x = fmaf(f, x.x, acc.x);
      acc.y = fmaf(f, x.y, acc.y);
      acc.z = fmaf(f, x.z, acc.z);
      acc.w = fmaf(f, x.w, acc.w);
      lsum = fmaf(f, ts.l[v][h], lsum);
    }
    float* part = part0 + h * head_stride;
    *reinterpret_cast<float4*>(part + 4 + c4) = acc;
    if ((tid & 31) == 0) {
      part[0] = M;
      part[1] = lsum;
    }
  }
}

// The same with the split layout of the workspace: (row, query head, split), the tail in
// split n_splits.
__device__ __forceinline__ void tail_partial(const __half* __restrict__ q, int32_t num_q_heads,
                                             int32_t num_kv_heads,
                                             const __half* __restrict__ k_tail,
                                             const __half* __restrict__ v_tail, int row, int sb,
                                             int g, int T, float qscale, int32_t n_splits,
                                             float* __restrict__ ws, TailSmem& ts) {
  const int G = num_q_heads / num_kv_heads;
  tail_partial_at(q, num_q_heads, num_kv_heads, k_tail, v_tail, row, sb, g, T, qscale,
                  ws + ((int64_t(row) * num_q_heads + int64_t(g) * G) * (n_splits + 1) + n_splits) *
                           kPartStride,
                  int64_t(n_splits + 1) * kPartStride, ts);
}

}  // namespace
}  // namespace kvarn

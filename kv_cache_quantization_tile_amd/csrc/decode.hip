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
// Codes enter the MFMA as normal float16 numbers 1 + code * 2^(b - 10): the code bits are
// masked into mantissa bits b.. under the exponent of 1.0, with b chosen per code position so
// that few shifts are needed (keys b = 2 or 6, values b = 6 or 8); the B operand carries the
// factor 2^(10 - b). The MFMA then returns sum_k B_k + sum_k B'_k code_k, and the column sum
// sum_k B_k is removed through the accumulator's initial value together with the zero-point
// term. Subnormal operands are avoided on purpose: the matrix core accumulates products of
// subnormal inputs with visibly less than float32 precision.
//
// Per page, each wave first derives the float32 factors it needs (2 channels and 2 tokens per
// lane) into its own LDS slot; every other lane then reads them with vector LDS loads. The two
// lanes of a high / low column pair split the work of building the B operands and of the
// softmax (rows 0,1 of each C fragment on the high lane, rows 2,3 on the low lane) and swap
// halves with bank-masked DPP moves. B operands are scaled by a power of two per page so that
// their largest float16 high part is near 2^14 (no overflow, full low-part precision).
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
// (ks, vs: the page's powers of two for the B operands.)
struct WaveMeta {
  float4 ka[kDim / 4], kb[kDim / 4];   // read 4 channels at a time
  float2 kt[kTile / 2], vp[kTile / 2], vz[kTile / 2];   // read 2 tokens at a time
  float4 vr[kDim / 4];
};

struct DecodeSmem {
  float m[4][8];
  float l[4][8];
  float acc[4][8][kDim];
  WaveMeta meta[4];
};

// Raw loads of one page: key codes (16 B per 16-token block at 4 bits, 8 B at 2), value
// codes (8 B per 16-channel block at 2 bits, 16 B at 4), and entries 2l, 2l+1 of the 4
// float16 metadata arrays of each record.
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

template <int KB, int VB>
struct PageRegs {
  typename KeyRec<KB>::Codes kc[8];
  typename ValRec<VB>::Codes vc[8];
  uint32_t km[4], vm[4];
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

template <int AUX, int KB, int VB>
__device__ __forceinline__ void load_meta(PageRegs<KB, VB>& t, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, const LaneOffsets& o) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
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
// below 2^14; vs does the same for the PV one).
template <int KB, int VB>
__device__ __forceinline__ void page_factors(const PageRegs<KB, VB>& t, WaveMeta& wm, int l,
                                             float maxq, float fk, float fv) {
  const float rk0 = lo_h(t.km[0]), rk1 = hi_h(t.km[0]);
  const float ka0 = rk0 * lo_h(t.km[2]) * fk, ka1 = rk1 * hi_h(t.km[2]) * fk;
  const float sv0 = lo_h(t.vm[1]), sv1 = hi_h(t.vm[1]);
  const float vp0 = sv0 * lo_h(t.vm[2]) * fv, vp1 = sv1 * hi_h(t.vm[2]) * fv;
  const float mka = wave_max(fmaxf(ka0, ka1));
  const float mvp = wave_max(fmaxf(vp0, vp1));
  const int eks = pow2_norm_exp(maxq * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mka))));
  const int evs = pow2_norm_exp(__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mvp))));
  const float ks = __builtin_ldexpf(1.f, eks), iks = __builtin_ldexpf(1.f, -eks);
  const float vs = __builtin_ldexpf(1.f, evs), ivs = __builtin_ldexpf(1.f, -evs);
  const float a0 = ka0 * ks, a1 = ka1 * ks;
  reinterpret_cast<float2*>(wm.ka)[l] = make_float2(a0, a1);
  reinterpret_cast<float2*>(wm.kb)[l] =
      make_float2(fmaf(ks * rk0, lo_h(t.km[3]), -a0), fmaf(ks * rk1, hi_h(t.km[3]), -a1));
  wm.kt[l] = make_float2(lo_h(t.km[1]) * iks, hi_h(t.km[1]) * iks);
  const float p0 = vp0 * vs, p1 = vp1 * vs;
  wm.vp[l] = make_float2(p0, p1);
  wm.vz[l] =
      make_float2(fmaf(vs * sv0, lo_h(t.vm[3]), -p0), fmaf(vs * sv1, hi_h(t.vm[3]), -p1));
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

// Exact attention over the T staged float16 tokens of (sequence sb, KV head g), raw space,
// for output row `row`, written as split n_splits of each query head's partials. Run by the
// extra split of decode_pages_kernel; wave w handles heads 2w, 2w+1 of the group; p_sm is
// 8 x 128 floats of LDS.
__device__ void tail_partial(const __half* __restrict__ q, int32_t num_q_heads,
                             int32_t num_kv_heads, const __half* __restrict__ k_tail,
                             const __half* __restrict__ v_tail, int row, int sb, int g, int T,
                             float qscale, int32_t n_splits, float* __restrict__ ws,
                             float (*p_sm)[kTile]) {
  const int G = num_q_heads / num_kv_heads;
  if (T == 0) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const __half* kt = k_tail + (int64_t(sb) * num_kv_heads + g) * kTile * kDim;
  const __half* vt = v_tail + (int64_t(sb) * num_kv_heads + g) * kTile * kDim;
  for (int hh = 2 * w; hh < 2 * w + 2; ++hh) {
    if (hh >= G) break;
    const int hq = g * G + hh;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q + (int64_t(row) * num_q_heads + hq) * kDim);
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
    float* part = ws + ((int64_t(row) * num_q_heads + hq) * (n_splits + 1) + n_splits) * kPartStride;
    *reinterpret_cast<float2*>(part + 4 + 2 * l) = make_float2(o0, o1);
    if (l == 0) {
      part[0] = mx;
      part[1] = ps;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// One workgroup: (output row, KV head g, split) = (blockIdx.x, y, z). Wave w handles page slots
// split * 4 * tpw + w + 4 k, k < tpw. Writes one partial (m, l, acc) per query head. With
// tail buffers the grid has one more split, n_splits, which computes the tail partial. The
// row's sequence, page slots and tail follow row_geometry. KB, VB: key and value code widths;
// AUX: cache policy of the page loads.
template <int KB, int VB, int AUX>
__global__ void __launch_bounds__(kThreads)
decode_pages_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                    int64_t pool_num_pages, const int32_t* __restrict__ block_table,
                    int32_t bt_stride, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    const int32_t* __restrict__ cu_q, int32_t batch, float qscale, int32_t tpw,
                    int32_t n_splits, int32_t split_base, const __half* __restrict__ k_tail,
                    const __half* __restrict__ v_tail, float tail_qscale,
                    float* __restrict__ ws) {
  __shared__ DecodeSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int split = split_base + blockIdx.z, g = blockIdx.y, b = blockIdx.x;   // b: output row
  const int G = num_q_heads / num_kv_heads;
  const RowGeom rg = row_geometry(b, seq_lens, max_seq_len, cu_q, batch);
  if (split == n_splits) {   // the extra split (launched only with tail buffers): the tail
    tail_partial(q, num_q_heads, num_kv_heads, k_tail, v_tail, b, rg.b, g, rg.tail_len,
                 tail_qscale, n_splits, ws, reinterpret_cast<float (*)[kTile]>(&sm.acc[0][0][0]));
    return;
  }
  const int n_full = rg.n_slots;      // page slots of this row (the last may be masked)
  const int slot0 = split * 4 * tpw;
  if (slot0 >= n_full) return;

  const int n = l & 15, gq = l >> 4;
  const int h = n & 7;
  const bool hi = n < 8;
  const int side = hi ? 0 : 2;          // first C row this lane finishes (rows side, side+1)
  const bool head_ok = h < G;
  // all ones on low-part lanes; opaque to the optimizer so that selections by it stay
  // single bit-selects instead of becoming variable vector indices
  uint32_t lo_mask = uint32_t(int32_t(uint32_t(l) << 28) >> 31);
  asm volatile("" : "+v"(lo_mask));

  // ---- q_rot = H q * softmax_scale * log2(e): channels 32 gq + j ---------------------
  // Each lane keeps the 16 channels whose B-operand entries it builds:
  // qo[4 s + j] = channel 32 gq + 8 s + 2 side + j.
  float qo[16];
  float maxq;   // computed below, once the first page loads are issued

  float m_run = -INFINITY, l_part = 0.f;
  float acc[8][4];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[bb][i] = 0.f;

  WaveMeta& wm = sm.meta[w];
  // key channel 2l + j: 4-bit keys: nibble pair v = l % 4 -> b = 2 (even v) or 6; 2-bit keys:
  // crumb pair parity l % 2 -> b = 8 or 6; value token 2l + j: C row (2l + j) % 4 -> pair
  // parity -> 2-bit values: b = 8 (rows 0,1) or 6 (rows 2,3); 4-bit values: b = 2 or 6
  const float fk = (l & 1) ? 16.f : (KB == 4 ? 256.f : 4.f);
  const float fv = (l & 1) ? 16.f : (VB == 2 ? 4.f : 256.f);

  const int32_t* bt_row = block_table + int64_t(rg.b) * bt_stride;
  auto page_of = [&](int slot) -> int64_t {
    if (slot >= n_full) return -1;
    const int32_t page = __builtin_amdgcn_readfirstlane(bt_row[slot]);
    return (page < 0 || page >= pool_num_pages) ? -1 : int64_t(page);
  };
  // record addresses are wave-uniform: their descriptors live in scalar registers
  auto uniform_ptr = [](const uint8_t* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo32 = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi32 = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    return reinterpret_cast<const uint8_t*>((uint64_t(hi32) << 32) | lo32);
  };
  const LaneOffsets lo{uint32_t(n * 64 + 16 * gq), uint32_t(n * 32 + 8 * gq), uint32_t(4 * l)};
  // record index page * num_kv_heads + g fits 32 bits (the pool's record count is checked
  // on the host); byte offsets are 32 x 32 -> 64-bit products
  // (the page id is re-read as a scalar here so that the offset arithmetic stays scalar)
  // A page id below 0 (no page) gives an empty descriptor: its loads return zeros without
  // touching memory, so the prefetches below need no branch.
  auto krec_of = [&](int64_t page) {
    const uint32_t ps = __builtin_amdgcn_readfirstlane(uint32_t(page < 0 ? 0 : page));
    const uint32_t r = ps * uint32_t(num_kv_heads) + uint32_t(g);
    return record_rsrc(uniform_ptr(k_pool + uint64_t(r) * uint32_t(KeyRec<KB>::kRecord)),
                       page < 0 ? 0 : KeyRec<KB>::kRecord);
  };
  auto vrec_of = [&](int64_t page) {
    const uint32_t ps = __builtin_amdgcn_readfirstlane(uint32_t(page < 0 ? 0 : page));
    const uint32_t r = ps * uint32_t(num_kv_heads) + uint32_t(g);
    return record_rsrc(uniform_ptr(v_pool + uint64_t(r) * uint32_t(ValRec<VB>::kRecord)),
                       page < 0 ? 0 : ValRec<VB>::kRecord);
  };
  // Processes the page held in t; each part of t is reloaded with page `next` as soon as
  // this page has consumed it, so the loads overlap the rest of the page's work. A page
  // that is not `valid` (its id is out of range) runs the same code and adds nothing: its
  // maximum stays -inf and its weights exp2(s - inf) are 0.
  auto process = [&](PageRegs<KB, VB>& t, int64_t next, bool valid, int lim) {
    // ---- page factors into the wave's LDS slot ------------------------------------------
    page_factors(t, wm, l, maxq, fk, fv);
    load_meta<AUX>(t, krec_of(next), vrec_of(next), lo);
    // LDS operations of one wave complete in order: the writes above land before the reads
    // below, and after the previous page's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- B operand of QK (q'' high / low), bias + column-sum correction ---------------
    H8 bq[4];
    float bias;
    {
      float bpart = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c4 = 8 * gq + 2 * s + (side >> 1);   // channels 4 c4 .. 4 c4 + 3
        const float4 ka = wm.ka[c4];
        const float4 kb = wm.kb[c4];
        const float* q4 = &qo[4 * s];
        bpart = fmaf(q4[0], kb.x, bpart);
        bpart = fmaf(q4[1], kb.y, bpart);
        bpart = fmaf(q4[2], kb.z, bpart);
        bpart = fmaf(q4[3], kb.w, bpart);
        uint32_t h01, l01, h23, l23;
        split_pk(q4[0] * ka.x, q4[1] * ka.y, h01, l01);
        split_pk(q4[2] * ka.z, q4[3] * ka.w, h23, l23);
        // dwords 0,1 = channels 0..3 of the 8 (built by the high lane), 2,3 = channels 4..7
        bq[s].u[0] = swap8_into<kLoBanks>(h01, l01);
        bq[s].u[1] = swap8_into<kLoBanks>(h23, l23);
        bq[s].u[2] = swap8_into<kHiBanks>(l01, h01);
        bq[s].u[3] = swap8_into<kHiBanks>(l23, h23);
      }
      bpart += dpp_f<kDppRowRor8>(bpart);
      bias = pick(lo_mask, 0.f, rows4_sum(bpart));   // added once: on the high columns
    }

    // ---- QK: this lane finishes rows side, side+1 of each fragment -------------------------
    float sc[8][2];
    {
      const float4v binit = {bias, bias, bias, bias};
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        float4v c = binit;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          H8 a;
          if constexpr (KB == 4) {
            const uint32_t dw[4] = {t.kc[tb].x, t.kc[tb].y, t.kc[tb].z, t.kc[tb].w};
#pragma unroll
            for (int v = 0; v < 4; ++v) a.u[v] = k_pair(dw[s], v);
          } else {   // word d = s / 2 holds k-steps 2d, 2d+1 in crumbs 4 (s % 2) + v (+ 8)
            const uint32_t word = (s >> 1) ? t.kc[tb].y : t.kc[tb].x;
#pragma unroll
            for (int v = 0; v < 4; ++v) a.u[v] = v_pair(word, 4 * (s & 1) + v);
          }
          c = mfma16x16x32(a.v, bq[s].v, c);
        }
        const float2 st = wm.kt[8 * tb + 2 * gq + (side >> 1)];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // high lane: own c[j] + partner c[j]; low lane: own c[2+j] + partner c[2+j]
          const float mine = pick(lo_mask, c[2 + j], c[j]);
          const float send = pick(lo_mask, c[j], c[2 + j]);
          sc[tb][j] = (mine + dpp_f<kDppRowRor8>(send)) * (j ? st.y : st.x);
        }
      }
    }
    load_kcodes<AUX>(t, krec_of(next), lo);
    if (lim < kTile) {   // a causally cut page: tokens from lim on do not count
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (16 * tb + 4 * gq + side + j >= lim) sc[tb][j] = -INFINITY;
    }

    // ---- online softmax ------------------------------------------------------------------
    float mt = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int tb = 1; tb < 8; ++tb) mt = fmaxf(mt, fmaxf(sc[tb][0], sc[tb][1]));
    mt = fmaxf(mt, dpp_f<kDppRowRor8>(mt));
    mt = rows4_max(mt);
    const float m_new = fmaxf(m_run, valid ? mt : -INFINITY);
    const float alpha = valid ? exp2_fast(m_run - m_new) : 1.f;
    const float m_sub = valid ? m_new : INFINITY;
    H8 bp[4];
    float vcorr;
    {
      float psum = 0.f, zpart = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t hh[2], ll[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tb = 2 * s + e;
          const int t2 = 8 * tb + 2 * gq + (side >> 1);   // tokens 2 t2, 2 t2 + 1
          const float2 vp = wm.vp[t2];
          const float2 vz = wm.vz[t2];
          const float p0 = exp2_fast(sc[tb][0] - m_sub), p1 = exp2_fast(sc[tb][1] - m_sub);
          psum += p0 + p1;
          zpart = fmaf(p0, vz.x, fmaf(p1, vz.y, zpart));
          split_pk(p0 * vp.x, p1 * vp.y, hh[e], ll[e]);
        }
        // dword 0 = rows 0,1 of fragment 2s (high lane built them), 1 = rows 2,3 (low lane),
        // 2, 3 the same for fragment 2s + 1
        bp[s].u[0] = swap8_into<kLoBanks>(hh[0], ll[0]);
        bp[s].u[1] = swap8_into<kHiBanks>(ll[0], hh[0]);
        bp[s].u[2] = swap8_into<kLoBanks>(hh[1], ll[1]);
        bp[s].u[3] = swap8_into<kHiBanks>(ll[1], hh[1]);
      }
      zpart += dpp_f<kDppRowRor8>(zpart);
      vcorr = pick(lo_mask, 0.f, rows4_sum(zpart));  // added once: on the high columns
      l_part = fmaf(l_part, alpha, psum);
    }
    m_run = m_new;

    // ---- PV ---------------------------------------------------------------------------
    if (!__all(alpha == 1.f)) {   // some head's running maximum moved: rescale in place
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[bb][i] *= alpha;
    }
    const float4v vinit = {vcorr, vcorr, vcorr, vcorr};
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      float4v c = vinit;
      if constexpr (VB == 2) {
        const uint2 vc = t.vc[bb];
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
      } else {   // word m = k-step m; nibbles v, 4 + v = its tokens 2v, 2v + 1
        const uint32_t words[4] = {t.vc[bb].x, t.vc[bb].y, t.vc[bb].z, t.vc[bb].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          H8 a;
#pragma unroll
          for (int v = 0; v < 4; ++v) a.u[v] = k_pair(words[m], v);
          c = mfma16x16x32(a.v, bp[m].v, c);
        }
      }
      const float4 rv = wm.vr[4 * bb + gq];
      acc[bb][0] = fmaf(rv.x, c[0], acc[bb][0]);
      acc[bb][1] = fmaf(rv.y, c[1], acc[bb][1]);
      acc[bb][2] = fmaf(rv.z, c[2], acc[bb][2]);
      acc[bb][3] = fmaf(rv.w, c[3], acc[bb][3]);
    }
    load_vcodes<AUX>(t, vrec_of(next), lo);
  };

  PageRegs<KB, VB> t;
  const int wslot = __builtin_amdgcn_readfirstlane(slot0 + w);   // this wave's first slot
  int64_t cur = page_of(wslot);
  load_meta<AUX>(t, krec_of(cur), vrec_of(cur), lo);
  load_kcodes<AUX>(t, krec_of(cur), lo);
  load_vcodes<AUX>(t, vrec_of(cur), lo);
  // q is rotated while the first page's loads are in flight
  {
    float qr[32];
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
    float mq = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      qr[j] *= qscale;  // includes 1/sqrt(128) of H
      mq = fmaxf(mq, fabsf(qr[j]));
    }
    maxq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(mq))));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) qo[4 * s + j] = hi ? qr[8 * s + j] : qr[8 * s + 4 + j];
  }
  // pages of this wave: slots wslot, wslot + 4, ... below n_full, at most tpw of them
  // (a loop with one exit keeps the running state in place across iterations)
  const int n_here = wslot < n_full ? min(tpw, (n_full - wslot + 3) >> 2) : 0;
  for (int k = 0; k < n_here; ++k) {
    const int64_t next = k + 1 < n_here ? page_of(wslot + 4 * (k + 1)) : -1;
    process(t, next, cur >= 0, wslot + 4 * k == n_full - 1 ? rg.mask_lim : kTile);
    cur = next;
  }

  // ---- combine the high / low columns, then the 4 waves --------------------------------
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[bb][i] += dpp_f<kDppRowRor8>(acc[bb][i]);
  l_part += dpp_f<kDppRowRor8>(l_part);
  const float l_run = rows4_sum(l_part);
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

// ---- multi-query read ------------------------------------------------------------------
//
// Many query rows per sequence: a wave holds 16 query vectors of one sequence and KV head,
// R = floor(16 / G) consecutive rows x the G heads of the group, one per MFMA column. The page
// walk, the per-page factors and the code unpacking are shared by the 16 queries; each
// query's own causal limit masks its scores. QK takes the key codes as the A operand and the
// scaled queries as B (C: 16 tokens x 16 queries); the float16 high and low parts of B are two
// MFMAs into the same accumulator, so the float32-level product needs no lane exchange. The
// softmax weights of a C fragment pair are already the PV B operand (the value record's token
// order), again as high + low parts; C of PV is 16 channels x 16 queries.
//
// Workgroups: the rows are cut into windows of 4R global row indices; workgroup j of the grid
// is window m of sequence b with j = m + b (a window that two sequences share appears once per
// sequence), found by a binary search over cu_q; wave w takes rows 4R m + R w .. + R - 1 of the
// window that belong to sequence b. grid: (ceil(rows / 4R) + batch, KV heads, splits [+ tail]).

struct MqSmem {
  WaveMeta meta[4];
  union {
    float4 q[4][8][64];   // q_rot per wave: [k][lane] = channels 32 gq + 4k .. 4k + 3
    float p[8][kTile];    // tail split: softmax weights of the staged tokens
  };
};

struct MqWindow {
  int b;          // sequence
  int r0, r1;     // its rows in this window: r0 .. r1 - 1 (r1 <= r0: none)
};

__device__ __forceinline__ MqWindow mq_window(int j, int rows_per_window,
                                              const int32_t* __restrict__ cu_q, int32_t batch,
                                              int32_t n_rows) {
  // the last b with floor(cu_q[b] / W) + b <= j
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] / rows_per_window + mid <= j) lo = mid; else hi = mid;
  }
  MqWindow r;
  r.b = lo;
  const int m = j - lo;
  const int64_t w0 = int64_t(m) * rows_per_window;
  int64_t a = cu_q[lo], e = cu_q[lo + 1];
  if (a < w0) a = w0;
  if (e > w0 + rows_per_window) e = w0 + rows_per_window;
  if (a < 0) a = 0;
  if (e > n_rows) e = n_rows;
  r.r0 = int(a);
  r.r1 = int(e);
  return r;
}

template <int KB, int VB>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mq_pages_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                int64_t pool_num_pages, const int32_t* __restrict__ block_table,
                int32_t bt_stride, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                const int32_t* __restrict__ cu_q, int32_t batch, int32_t n_rows, float qscale,
                int32_t slots_per_split, int32_t n_splits, int32_t split_base,
                const __half* __restrict__ k_tail, const __half* __restrict__ v_tail,
                float tail_qscale, float* __restrict__ ws) {
  __shared__ MqSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int split = split_base + blockIdx.z, g = blockIdx.y;
  const int G = num_q_heads / num_kv_heads;
  const int R = 16 / G;                                   // rows per wave
  const MqWindow win = mq_window(blockIdx.x, 4 * R, cu_q, batch, n_rows);
  if (split == n_splits) {   // the tails of the window's rows, one row after the other
    for (int row = win.r0; row < win.r1; ++row) {   // uniform over the workgroup
      const RowGeom rgr = row_geometry(row, seq_lens, max_seq_len, cu_q, batch);
      tail_partial(q, num_q_heads, num_kv_heads, k_tail, v_tail, row, rgr.b, g, rgr.tail_len,
                   tail_qscale, n_splits, ws, sm.p);
      __syncthreads();
    }
    return;
  }
  // (no workgroup barrier past this point: waves leave on their own)
  const int wr0 = __builtin_amdgcn_readfirstlane(win.r0 + R * w);   // this wave's rows
  const int wr1 = __builtin_amdgcn_readfirstlane(min(win.r1, wr0 + R));
  if (wr0 >= wr1) return;
  // pages: the slots of the wave's last row (the longest), within this split
  const RowGeom rg_last = row_geometry(wr1 - 1, seq_lens, max_seq_len, cu_q, batch);
  const RowGeom rg_first = row_geometry(wr0, seq_lens, max_seq_len, cu_q, batch);
  const int s0 = __builtin_amdgcn_readfirstlane(split * slots_per_split);
  const int s1 = __builtin_amdgcn_readfirstlane(min(s0 + slots_per_split, rg_last.n_slots));
  if (s0 >= s1) return;
  // tokens of the pages that every row of the wave attends to (no masking below this)
  const int lp_min = __builtin_amdgcn_readfirstlane(
      rg_first.n_slots > 0 ? kTile * (rg_first.n_slots - 1) + rg_first.mask_lim : 0);

  const int n = l & 15, gq = l >> 4;
  const int rl = n / G, hh = n - rl * G;        // this column: row wr0 + rl, head hh
  const bool col_ok = wr0 + rl < wr1;
  const int row = col_ok ? wr0 + rl : wr0;
  // tokens of this column's row held in pages (the rest, if any, is its staged tail)
  int lp_col = 0;
  if (col_ok) {
    const RowGeom rgc = row_geometry(row, seq_lens, max_seq_len, cu_q, batch);
    lp_col = rgc.n_slots > 0 ? kTile * (rgc.n_slots - 1) + rgc.mask_lim : 0;
  }

  WaveMeta& wm = sm.meta[w];
  const float fk = (l & 1) ? 16.f : (KB == 4 ? 256.f : 4.f);
  const float fv = (l & 1) ? 16.f : (VB == 2 ? 4.f : 256.f);
  const int32_t* bt_row = block_table + int64_t(rg_last.b) * bt_stride;
  auto page_of = [&](int slot) -> int64_t {
    if (slot >= s1) return -1;
    const int32_t page = __builtin_amdgcn_readfirstlane(bt_row[slot]);
    return (page < 0 || page >= pool_num_pages) ? -1 : int64_t(page);
  };
  auto uniform_ptr = [](const uint8_t* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo32 = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi32 = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    return reinterpret_cast<const uint8_t*>((uint64_t(hi32) << 32) | lo32);
  };
  const LaneOffsets lo{uint32_t(n * 64 + 16 * gq), uint32_t(n * 32 + 8 * gq), uint32_t(4 * l)};
  auto krec_of = [&](int64_t page) {
    const uint32_t ps = __builtin_amdgcn_readfirstlane(uint32_t(page < 0 ? 0 : page));
    const uint32_t r = ps * uint32_t(num_kv_heads) + uint32_t(g);
    return record_rsrc(uniform_ptr(k_pool + uint64_t(r) * uint32_t(KeyRec<KB>::kRecord)),
                       page < 0 ? 0 : KeyRec<KB>::kRecord);
  };
  auto vrec_of = [&](int64_t page) {
    const uint32_t ps = __builtin_amdgcn_readfirstlane(uint32_t(page < 0 ? 0 : page));
    const uint32_t r = ps * uint32_t(num_kv_heads) + uint32_t(g);
    return record_rsrc(uniform_ptr(v_pool + uint64_t(r) * uint32_t(ValRec<VB>::kRecord)),
                       page < 0 ? 0 : ValRec<VB>::kRecord);
  };

  PageRegs<KB, VB> t;
  int64_t cur = page_of(s0);
  load_meta<kReuseLoad>(t, krec_of(cur), vrec_of(cur), lo);
  load_kcodes<kReuseLoad>(t, krec_of(cur), lo);
  load_vcodes<kReuseLoad>(t, vrec_of(cur), lo);

  // ---- q_rot of this column: channels 32 gq + j (the 4 lanes of a column hold 128), kept
  // in LDS (registers are the page loop's)
  float maxq;
  {
    float qr[32];
    const __half* qrow = q + (int64_t(row) * num_q_heads + int64_t(g) * G + hh) * kDim + 32 * gq;
#pragma unroll
    for (int k = 0; k < 4; ++k) load_h8(reinterpret_cast<const uint8_t*>(qrow + 8 * k), &qr[8 * k]);
    if (!col_ok) {
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
    float mq = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      qr[j] *= qscale;  // includes 1/sqrt(128) of H
      mq = fmaxf(mq, fabsf(qr[j]));
    }
    maxq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(mq))));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      sm.q[w][k][l] = make_float4(qr[4 * k], qr[4 * k + 1], qr[4 * k + 2], qr[4 * k + 3]);
  }

  float m_run = -INFINITY, l_part = 0.f;
  float acc[8][4];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[bb][i] = 0.f;

  for (int slot = s0; slot < s1; ++slot) {
    const int64_t next = page_of(slot + 1);
    const bool valid = cur >= 0;
    page_factors(t, wm, l, maxq, fk, fv);
    load_meta<kReuseLoad>(t, krec_of(next), vrec_of(next), lo);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- B operand of QK: q_rot * ka (high, low), bias = q_rot . kb ---------------------
    H8 bqh[4], bql[4];
    float bias;
    {
      float bpart = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float4 ka0 = wm.ka[8 * gq + 2 * s], ka1 = wm.ka[8 * gq + 2 * s + 1];
        const float4 kb0 = wm.kb[8 * gq + 2 * s], kb1 = wm.kb[8 * gq + 2 * s + 1];
        const float4 q0 = sm.q[w][2 * s][l], q1 = sm.q[w][2 * s + 1][l];
        const float ka[8] = {ka0.x, ka0.y, ka0.z, ka0.w, ka1.x, ka1.y, ka1.z, ka1.w};
        const float kb[8] = {kb0.x, kb0.y, kb0.z, kb0.w, kb1.x, kb1.y, kb1.z, kb1.w};
        const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float x0 = qv[2 * d], x1 = qv[2 * d + 1];
          bpart = fmaf(x0, kb[2 * d], fmaf(x1, kb[2 * d + 1], bpart));
          split_pk(x0 * ka[2 * d], x1 * ka[2 * d + 1], bqh[s].u[d], bql[s].u[d]);
        }
      }
      bias = rows4_sum(bpart);
    }

    // ---- QK: C rows = tokens 16 tb + 4 gq + i, column = this lane's query ----------------
    float sc[8][4];
    {
      const float4v binit = {bias, bias, bias, bias};
      const float* kt = reinterpret_cast<const float*>(wm.kt);
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        float4v c = binit;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          H8 a;
          if constexpr (KB == 4) {
            const uint32_t dw[4] = {t.kc[tb].x, t.kc[tb].y, t.kc[tb].z, t.kc[tb].w};
#pragma unroll
            for (int v = 0; v < 4; ++v) a.u[v] = k_pair(dw[s], v);
          } else {
            const uint32_t word = (s >> 1) ? t.kc[tb].y : t.kc[tb].x;
#pragma unroll
            for (int v = 0; v < 4; ++v) a.u[v] = v_pair(word, 4 * (s & 1) + v);
          }
          c = mfma16x16x32(a.v, bqh[s].v, c);
          c = mfma16x16x32(a.v, bql[s].v, c);
        }
        const float4 st = *reinterpret_cast<const float4*>(kt + 16 * tb + 4 * gq);
        sc[tb][0] = c[0] * st.x;
        sc[tb][1] = c[1] * st.y;
        sc[tb][2] = c[2] * st.z;
        sc[tb][3] = c[3] * st.w;
      }
    }
    load_kcodes<kReuseLoad>(t, krec_of(next), lo);
    if (kTile * (slot + 1) > lp_min) {   // some column's limit falls inside this page
      const int lim = lp_col - kTile * slot;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tb + 4 * gq + i >= lim) sc[tb][i] = -INFINITY;
    }

    // ---- online softmax (per column) -------------------------------------------------------
    float mt = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[tb][i]);
    mt = rows4_max(mt);
    const float m_new = valid ? fmaxf(m_run, mt) : m_run;
    const bool live = valid && m_new != -INFINITY;
    const float alpha = live ? exp2_fast(m_run - m_new) : 1.f;
    const float m_sub = live ? m_new : INFINITY;
    H8 bph[4], bpl[4];
    float vcorr;
    {
      float psum = 0.f, zpart = 0.f;
      const float* vp = reinterpret_cast<const float*>(wm.vp);
      const float* vz = reinterpret_cast<const float*>(wm.vz);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tb = 2 * s + e;
          const float4 vp4 = *reinterpret_cast<const float4*>(vp + 16 * tb + 4 * gq);
          const float4 vz4 = *reinterpret_cast<const float4*>(vz + 16 * tb + 4 * gq);
          const float p0 = exp2_fast(sc[tb][0] - m_sub), p1 = exp2_fast(sc[tb][1] - m_sub);
          const float p2 = exp2_fast(sc[tb][2] - m_sub), p3 = exp2_fast(sc[tb][3] - m_sub);
          psum += (p0 + p1) + (p2 + p3);
          zpart = fmaf(p0, vz4.x, fmaf(p1, vz4.y, fmaf(p2, vz4.z, fmaf(p3, vz4.w, zpart))));
          split_pk(p0 * vp4.x, p1 * vp4.y, bph[s].u[2 * e], bpl[s].u[2 * e]);
          split_pk(p2 * vp4.z, p3 * vp4.w, bph[s].u[2 * e + 1], bpl[s].u[2 * e + 1]);
        }
      }
      vcorr = rows4_sum(zpart);
      l_part = fmaf(l_part, alpha, psum);
    }
    m_run = m_new;

    // ---- PV: C rows = channels 16 bb + 4 gq + i ---------------------------------------------
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[bb][i] *= alpha;
    }
    const float4v vinit = {vcorr, vcorr, vcorr, vcorr};
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      float4v c = vinit;
      if constexpr (VB == 2) {
        const uint2 vc = t.vc[bb];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t word = d ? vc.y : vc.x;
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            H8 a;
#pragma unroll
            for (int v = 0; v < 4; ++v) a.u[v] = v_pair(word, 4 * hs + v);
            c = mfma16x16x32(a.v, bph[2 * d + hs].v, c);
            c = mfma16x16x32(a.v, bpl[2 * d + hs].v, c);
          }
        }
      } else {
        const uint32_t words[4] = {t.vc[bb].x, t.vc[bb].y, t.vc[bb].z, t.vc[bb].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          H8 a;
#pragma unroll
          for (int v = 0; v < 4; ++v) a.u[v] = k_pair(words[m], v);
          c = mfma16x16x32(a.v, bph[m].v, c);
          c = mfma16x16x32(a.v, bpl[m].v, c);
        }
      }
      const float4 rv = wm.vr[4 * bb + gq];
      acc[bb][0] = fmaf(rv.x, c[0], acc[bb][0]);
      acc[bb][1] = fmaf(rv.y, c[1], acc[bb][1]);
      acc[bb][2] = fmaf(rv.z, c[2], acc[bb][2]);
      acc[bb][3] = fmaf(rv.w, c[3], acc[bb][3]);
    }
    load_vcodes<kReuseLoad>(t, vrec_of(next), lo);
    cur = next;
  }

  // ---- this column's partial: m, l, acc (channels 16 bb + 4 gq + i) -------------------------
  const float l_run = rows4_sum(l_part);
  if (col_ok) {
    float* part = ws + ((int64_t(row) * num_q_heads + int64_t(g) * G + hh) * (n_splits + 1) + split) * kPartStride;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
      *reinterpret_cast<float4*>(part + 4 + 16 * bb + 4 * gq) =
          make_float4(acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]);
    if (gq == 0) {
      part[0] = m_run;
      part[1] = l_run;
    }
  }
}

// Merge the splits of one (sequence, query head): log-sum-exp weights, H^T on the page
// part (rotated space), plus the raw-space tail; float16 output. One 256-thread workgroup
// per (pair of query heads, sequence): 128 threads per head, thread c owns channel c; split
// weights are computed once in LDS, then every thread streams its channel of all partials
// (independent loads). (Pairs halve the workgroup count of a many-row read.)
__global__ void __launch_bounds__(256)
decode_merge_kernel(int32_t num_q_heads, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    const int32_t* __restrict__ cu_q, int32_t batch, int32_t tiles_per_split,
                    int32_t n_splits, int32_t has_tail, const float* __restrict__ ws,
                    __half* __restrict__ out) {
  __shared__ float wsh_[2][kMaxMergeSplits + 1];
  __shared__ float red_[2][2][2];
  __shared__ float xs_[2][kDim];
  const int pair = threadIdx.x >> 7;
  float* wsh = wsh_[pair];
  float (*red)[2] = red_[pair];
  float* xs = xs_[pair];
  // a head past the last (odd head count) runs along for the barriers and stores nothing
  const int hq = min(2 * int(blockIdx.x) + pair, num_q_heads - 1);
  const bool head_ok = 2 * int(blockIdx.x) + pair < num_q_heads;
  const int b = blockIdx.y;   // b: output row
  const int c = threadIdx.x & 127, lane = c & 63, wv = c >> 6;
  const RowGeom rg = row_geometry(b, seq_lens, max_seq_len, cu_q, batch);
  const int used = (rg.n_slots + tiles_per_split - 1) / tiles_per_split;
  const bool tail = has_tail && rg.tail_len != 0;
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
  if (head_ok) out[(int64_t(b) * num_q_heads + hq) * kDim + c] = __float2half_rn(a * inv);
}

}  // namespace

int32_t decode_tiles_per_wave(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t max_full = max_seq_len / kTile;
  const int64_t work = int64_t(batch) * num_kv_heads * max_full;
  // one round of waves over the chip: 256 CUs x 8 resident waves (2 per SIMD)
  int64_t tpw = (work + 2047) / 2048;
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

// Multi-query read: page slots per split, so that the waves (16 query vectors each) fill the
// chip for about eight rounds of its 2048 resident waves, with at least 8 pages per split.
int32_t mq_slots_per_split(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t max_seq_len) {
  const int64_t max_full = max_seq_len / kTile;
  if (max_full <= 0) return 1;
  const int64_t R = 16 / (num_q_heads / num_kv_heads);
  const int64_t waves = ((int64_t(rows) + R - 1) / R) * num_kv_heads;
  int64_t ns = (8 * 2048 + waves - 1) / waves;
  const int64_t cap = (max_full + 7) / 8;
  if (ns > cap) ns = cap;
  if (ns > kMaxMergeSplits) ns = kMaxMergeSplits;
  if (ns < 1) ns = 1;
  return int32_t((max_full + ns - 1) / ns);
}

int32_t mq_num_splits(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t max_seq_len) {
  const int32_t max_full = max_seq_len / kTile;
  const int32_t per = mq_slots_per_split(rows, num_q_heads, num_kv_heads, max_seq_len);
  const int32_t ns = (max_full + per - 1) / per;
  return ns < 1 ? 1 : ns;
}

size_t chunk_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t max_seq_len) {
  // either layout may run (one row per sequence keeps the decode's)
  int32_t ns = decode_num_splits(rows, num_kv_heads, max_seq_len);
  const int32_t nm = mq_num_splits(rows, num_q_heads, num_kv_heads, max_seq_len);
  if (nm > ns) ns = nm;
  return size_t(rows) * num_q_heads * (ns + 1) * kPartStride * sizeof(float);
}

hipError_t launch_decode(int k_bits, int v_bits, const void* q, int32_t rows,
                         int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                         const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                         const int32_t* cu_q, int32_t batch, const void* k_tail,
                         const void* v_tail, float softmax_scale, void* workspace, void* out,
                         hipStream_t stream) {
  // several query rows of one sequence (more rows than sequences): the multi-query kernel
  const bool multi_row = cu_q != nullptr && rows > batch;
  const int32_t tpw = decode_tiles_per_wave(rows, num_kv_heads, max_seq_len);
  const int32_t per_split =
      multi_row ? mq_slots_per_split(rows, num_q_heads, num_kv_heads, max_seq_len) : 4 * tpw;
  const int32_t ns = multi_row ? mq_num_splits(rows, num_q_heads, num_kv_heads, max_seq_len)
                               : decode_num_splits(rows, num_kv_heads, max_seq_len);
  const float qscale = softmax_scale * kLog2e;
  float* ws = static_cast<float*>(workspace);
  const bool has_tail = k_tail != nullptr && v_tail != nullptr;
  // page splits (only if a full page can exist) plus, with tail buffers, one tail split
  const int32_t n_split_wg = (max_seq_len >= kTile ? ns : 0) + (has_tail ? 1 : 0);
  if (n_split_wg > 0) {
    // without pages the only split launched is the tail, which must land on index ns
    const int32_t first = max_seq_len >= kTile ? 0 : ns;
    // rows fastest, splits slowest: workgroups are dealt to the 8 XCDs round-robin in linear
    // order, so consecutive ones must all carry work (a split axis of period 2, pages +
    // tail, would leave every page workgroup on the even XCDs)
    const hipError_t e = with_preset(k_bits, v_bits, [&](auto kb, auto vb) {
      constexpr int KB = decltype(kb)::value, VB = decltype(vb)::value;
      if (multi_row) {   // 16 query vectors per wave, windows of 4R rows per workgroup
        const int R = 16 / (num_q_heads / num_kv_heads);
        hipLaunchKernelGGL((mq_pages_kernel<KB, VB>),
                           dim3((rows + 4 * R - 1) / (4 * R) + batch, num_kv_heads, n_split_wg),
                           dim3(kThreads), 0, stream, static_cast<const __half*>(q), num_q_heads,
                           num_kv_heads, static_cast<const uint8_t*>(k_pool),
                           static_cast<const uint8_t*>(v_pool), pool_num_pages, block_table,
                           bt_stride, seq_lens, max_seq_len, cu_q, batch, rows,
                           qscale * kInvSqrt128, per_split, ns, first,
                           static_cast<const __half*>(k_tail), static_cast<const __half*>(v_tail),
                           qscale, ws);
        return;
      }
      // decode streams every page once; a read with one query per sequence reuses them
      auto kernel = cu_q ? decode_pages_kernel<KB, VB, kReuseLoad>
                         : decode_pages_kernel<KB, VB, kStreamLoad>;
      hipLaunchKernelGGL(kernel, dim3(rows, num_kv_heads, n_split_wg), dim3(kThreads), 0, stream,
                         static_cast<const __half*>(q), num_q_heads, num_kv_heads,
                         static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool),
                         pool_num_pages, block_table, bt_stride, seq_lens, max_seq_len, cu_q,
                         batch, qscale * kInvSqrt128, tpw, ns, first,
                         static_cast<const __half*>(k_tail), static_cast<const __half*>(v_tail),
                         qscale, ws);
    });
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_merge_kernel, dim3((num_q_heads + 1) / 2, rows), dim3(256), 0, stream,
                     num_q_heads, seq_lens, max_seq_len, cu_q, batch, per_split, ns,
                     has_tail ? 1 : 0, static_cast<const float*>(ws), static_cast<__half*>(out));
  return hipGetLastError();
}

}  // namespace kvarn

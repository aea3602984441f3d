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
#include <mutex>

#include "decode_common.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

template <int NG>
struct DecodeSmem {
  float m[4][8];
  float l[4][8];
  float acc[4][8][kDim];
  WaveMeta<NG> meta[4];
  int32_t pref[kMaxBalancedRows + 1];   // balanced layout: full pages before each sequence
  int32_t wsum[4];
};

// Split layout (BAL = false): one workgroup per (output row b, KV head g, split) =
// (blockIdx.x / Hkv, blockIdx.x % Hkv, blockIdx.y). Wave w handles page slots
// split * 4 * tpw + w + 4 k, k < tpw. Writes one partial (m, l, acc) per query head. With
// tail buffers the grid has one more split, n_splits, which computes the tail partial. The
// row's sequence, page slots and tail follow row_geometry.
// Balanced layout (BAL = true; one query row per sequence): the full pages of all (sequence,
// KV head) segments, in order b, g, page, are one list of T pages, and wave i < W =
// min(4 n_page_wg, T) streams list entries [floor(i T / W), floor((i + 1) T / W)) (at least
// one), crossing segment boundaries; it writes one partial per segment it touches, at slot
// i + (b Hkv + g). Ragged lengths then cost no idle waves. Workgroup 0 also stores the page
// prefix sums for the merge. Workgroups n_page_wg.. are the tails, one per (b, g).
// KB, VB: key and value code widths; AUX: cache policy of the page loads.
template <int KB, int VB, int FMT, int NG, int AUX, bool BAL>
__global__ void __launch_bounds__(kThreads)
decode_pages_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                    int64_t pool_num_pages, const int32_t* __restrict__ block_table,
                    int32_t bt_stride, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    const int32_t* __restrict__ cu_q, int32_t batch, float qscale, int32_t tpw,
                    int32_t n_splits, int32_t split_base, const __half* __restrict__ k_tail,
                    const __half* __restrict__ v_tail, float tail_qscale,
                    float* __restrict__ ws, int32_t n_page_wg) {
  __shared__ DecodeSmem<NG> sm;
  static_assert(sizeof(DecodeSmem<NG>) >= sizeof(TailSmem), "the tail reuses the LDS");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int G = num_q_heads / num_kv_heads;
  // split layout: KV heads fastest, so that the workgroups dealt to the 8 XCDs round-robin in
  // linear order give each XCD the same heads of every sequence
  int split = 0, g = 0, b = 0;   // b: output row
  if constexpr (BAL) {
    if (int(blockIdx.x) >= n_page_wg) {   // a tail workgroup
      const int k = int(blockIdx.x) - n_page_wg;
      g = k % num_kv_heads;
      b = k / num_kv_heads;
      const RowGeom rt = row_geometry(b, seq_lens, max_seq_len, nullptr, batch);
      tail_partial_at(q, num_q_heads, num_kv_heads, k_tail, v_tail, b, b, g, rt.tail_len,
                      tail_qscale,
                      ws + balanced_tail_offset(n_page_wg, batch, num_q_heads, num_kv_heads) +
                          (int64_t(b) * num_q_heads + int64_t(g) * G) * kPartStride,
                      kPartStride, *reinterpret_cast<TailSmem*>(&sm));
      return;
    }
  } else {
    split = split_base + blockIdx.y;
    g = int(blockIdx.x) % num_kv_heads;
    b = int(blockIdx.x) / num_kv_heads;
  }
  const RowGeom rg = row_geometry(b, seq_lens, max_seq_len, cu_q, batch);
  if constexpr (!BAL) {
    if (split == n_splits) {   // the extra split (launched only with tail buffers): the tail
      tail_partial(q, num_q_heads, num_kv_heads, k_tail, v_tail, b, rg.b, g, rg.tail_len,
                   tail_qscale, n_splits, ws, *reinterpret_cast<TailSmem*>(&sm));
      return;
    }
  }
  const int n_full = rg.n_slots;      // page slots of this row (the last may be masked)
  const int slot0 = split * 4 * tpw;
  if constexpr (!BAL) {
    if (slot0 >= n_full) return;
  }

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

  WaveMeta<NG>& wm = sm.meta[w];
  // key channel 2l + j: 4-bit keys: nibble pair v = l % 4 -> b = 2 (even v) or 6; 2-bit keys:
  // crumb pair parity l % 2 -> b = 8 or 6; value token 2l + j: C row (2l + j) % 4 -> pair
  // parity -> 2-bit values: b = 8 (rows 0,1) or 6 (rows 2,3); 4-bit values: b = 2 or 6
  const float fk = (l & 1) ? 16.f : (KB == 4 ? 256.f : 4.f);
  const float fv = (l & 1) ? 16.f : (VB == 2 ? 4.f : 256.f);

  // record index of page slot `slot` (< n_slots) of block-table row bt_r for KV head gg, or -1
  // (no slot, or a page outside the pool)
  auto rec_of = [&](const int32_t* bt_r, int slot, int n_slots, int gg) -> int64_t {
    if (slot >= n_slots) return -1;
    const int32_t page = __builtin_amdgcn_readfirstlane(bt_r[slot]);
    return (page < 0 || page >= pool_num_pages) ? -1 : int64_t(page) * num_kv_heads + gg;
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
  // (the index is re-read as a scalar here so that the offset arithmetic stays scalar)
  // A record index below 0 (no page) gives an empty descriptor: its loads return zeros
  // without touching memory, so the prefetches below need no branch.
  auto krec_of = [&](int64_t rec) {
    const uint32_t r = __builtin_amdgcn_readfirstlane(uint32_t(rec < 0 ? 0 : rec));
    return record_rsrc(uniform_ptr(k_pool + uint64_t(r) * uint32_t(key_record<KB, FMT, NG>())),
                       rec < 0 ? 0 : key_record<KB, FMT, NG>());
  };
  auto vrec_of = [&](int64_t rec) {
    const uint32_t r = __builtin_amdgcn_readfirstlane(uint32_t(rec < 0 ? 0 : rec));
    return record_rsrc(uniform_ptr(v_pool + uint64_t(r) * uint32_t(val_record<VB, FMT, NG>())),
                       rec < 0 ? 0 : val_record<VB, FMT, NG>());
  };
  // Processes the page held in t; each part of t is reloaded with page `next` as soon as
  // this page has consumed it, so the loads overlap the rest of the page's work. A page
  // that is not `valid` (its id is out of range) runs the same code and adds nothing: its
  // maximum stays -inf and its weights exp2(s - inf) are 0.
  auto process = [&](PageRegs<KB, VB>& t, int64_t next, bool valid, int lim) {
    // ---- page factors into the wave's LDS slot ------------------------------------------
    page_factors<FMT, NG>(t, wm, l, maxq, fk, fv);
    load_meta<AUX, FMT, NG>(t, krec_of(next), vrec_of(next), lo);
    // LDS operations of one wave complete in order: the writes above land before the reads
    // below, and after the previous page's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- QK, per key group (NG = 2: token blocks 0..3 take the factors of tokens 0..63,
    // blocks 4..7 those of tokens 64..127): the B operand (q'' high / low) and the bias +
    // column-sum correction of the group, then its token blocks; this lane finishes rows
    // side, side+1 of each fragment
    float sc[8][2];
#pragma unroll
    for (int hq = 0; hq < NG; ++hq) {
      H8 bq[4];
      float bias;
      {
        float bpart = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c4 = 8 * gq + 2 * s + (side >> 1);   // channels 4 c4 .. 4 c4 + 3
          const float4 ka = wm.ka[hq][c4];
          const float4 kb = wm.kb[hq][c4];
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
      const float4v binit = {bias, bias, bias, bias};
#pragma unroll
      for (int tb = 8 / NG * hq; tb < 8 / NG * (hq + 1); ++tb) {
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
    // B operand of PV for value group hv (the softmax weights times the group's value
    // factors, high / low) and its zero-point correction. NG = 1 turns the scores into
    // weights here, adding them to psum; NG = 2 reads weights computed beforehand.
    auto pv_operands = [&](int hv, H8 (&bp)[4], float& psum) -> float {
      float zpart = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t hh[2], ll[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tb = 2 * s + e;
          const int t2 = 8 * tb + 2 * gq + (side >> 1);   // tokens 2 t2, 2 t2 + 1
          const float2 vp = wm.vp[hv][t2];
          const float2 vz = wm.vz[hv][t2];
          float p0 = sc[tb][0], p1 = sc[tb][1];
          if constexpr (NG == 1) {
            p0 = exp2_fast(p0 - m_sub);
            p1 = exp2_fast(p1 - m_sub);
            psum += p0 + p1;
          }
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
      return pick(lo_mask, 0.f, rows4_sum(zpart));  // added once: on the high columns
    };
    // PV of channel blocks bb0 .. bb0 + 8 / NG - 1 (one value group)
    auto pv_blocks = [&](const H8 (&bp)[4], float vcorr, int bb0) {
      const float4v vinit = {vcorr, vcorr, vcorr, vcorr};
#pragma unroll
      for (int k = 0; k < 8 / NG; ++k) {
        const int bb = bb0 + k;
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
    };
    auto rescale = [&]() {
      if (!__all(alpha == 1.f)) {   // some head's running maximum moved: rescale in place
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[bb][i] *= alpha;
      }
    };
    // ---- softmax weights and PV (NG = 2: channel blocks 0..3 take the value factors of
    // channels 0..63, blocks 4..7 those of channels 64..127) --------------------------------
    if constexpr (NG == 1) {
      H8 bp[4];
      float psum = 0.f;
      const float vcorr = pv_operands(0, bp, psum);
      l_part = fmaf(l_part, alpha, psum);
      m_run = m_new;
      rescale();
      pv_blocks(bp, vcorr, 0);
    } else {
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        sc[tb][0] = exp2_fast(sc[tb][0] - m_sub);
        sc[tb][1] = exp2_fast(sc[tb][1] - m_sub);
        psum += sc[tb][0] + sc[tb][1];
      }
      l_part = fmaf(l_part, alpha, psum);
      m_run = m_new;
      rescale();
#pragma unroll
      for (int hv = 0; hv < NG; ++hv) {
        H8 bp[4];
        const float vcorr = pv_operands(hv, bp, psum);
        pv_blocks(bp, vcorr, 8 / NG * hv);
      }
    }
    load_vcodes<AUX>(t, vrec_of(next), lo);
  };

  // q_rot = H q * softmax_scale * log2(e) of (output row bq, KV head gh) into qo, maxq
  // (split in two: the loads of a wave's first q go out before its first page's, so that the
  // rotation waits for q alone, not for the page queued ahead of it)
  auto q_loads = [&](int bq, int gh, uint4 (&raw)[4]) {
    const __half* qrow = q + (int64_t(bq) * num_q_heads + int64_t(gh) * G + (head_ok ? h : 0)) * kDim + 32 * gq;
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = *reinterpret_cast<const uint4*>(qrow + 8 * k);
  };
  auto rotate_loaded_q = [&](const uint4 (&raw)[4]) {
    float qr[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qr[8 * k + 2 * e] = h2f(uint16_t(wd[e] & 0xFFFF));
        qr[8 * k + 2 * e + 1] = h2f(uint16_t(wd[e] >> 16));
      }
    }
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
  };
  // the high / low column partners' accumulators and row sums added up: acc on every lane,
  // the head's l returned
  auto combine_columns = [&]() {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[bb][i] += dpp_f<kDppRowRor8>(acc[bb][i]);
    l_part += dpp_f<kDppRowRor8>(l_part);
    return rows4_sum(l_part);
  };

  PageRegs<KB, VB> t;
  if constexpr (BAL) {
    // ---- full pages of every sequence and their prefix sums, in LDS ---------------------
    {
      const int per = (batch + kThreads - 1) / kThreads;   // <= 4 (batch <= kMaxBalancedRows)
      int cnt[4], run = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = tid * per + k;
        int v = 0;
        if (k < per && i < batch) {
          int32_t L = seq_lens[i];
          L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
          v = L / kTile;
        }
        cnt[k] = v;
        run += v;
      }
      int incl = run;   // inclusive scan over the wave
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (l >= off) incl += y;
      }
      if (l == 63) sm.wsum[w] = incl;
      __syncthreads();
      int excl = incl - run;
      for (int ww = 0; ww < w; ++ww) excl += sm.wsum[ww];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = tid * per + k;
        if (k < per && i < batch) {
          sm.pref[i] = excl;
          excl += cnt[k];
        }
      }
      if (tid == 0) sm.pref[batch] = sm.wsum[0] + sm.wsum[1] + sm.wsum[2] + sm.wsum[3];
      __syncthreads();
      if (blockIdx.x == 0) {   // for the merge
        int32_t* wp = reinterpret_cast<int32_t*>(
            ws + balanced_pref_offset(n_page_wg, batch, num_q_heads, num_kv_heads));
        for (int i = tid; i <= batch; i += kThreads) wp[i] = sm.pref[i];
      }
    }
    // (no workgroup barrier past this point: waves leave on their own)
    // list of T pages (< 2^31, checked on the host), spread over min(4 n_page_wg, T) waves
    const int T = __builtin_amdgcn_readfirstlane(num_kv_heads * sm.pref[batch]);
    const int n_waves = min(4 * n_page_wg, T);
    const int wi = __builtin_amdgcn_readfirstlane(4 * int(blockIdx.x) + w);   // wave-uniform
    if (wi >= n_waves) return;
    int64_t x = int64_t(T) * wi / n_waves;
    const int64_t x_end = int64_t(T) * (wi + 1) / n_waves;
    // Issue priority by progress: 3 in the first quarter of this wave's pages, down to 0 in
    // the last. The waves that share a SIMD then keep pace with each other (the one behind
    // wins the issue arbitration) instead of one finishing first and leaving the other alone.
    // With the wave's n entries starting at x0, quarter k starts at entry x0 + ceil(k n / 4),
    // the first entry xc with floor(4 (xc - x0) / n) >= k: three bounds found once instead of
    // a 64-bit division per page.
    const int64_t n_mine = x_end - x;
    const int64_t quarter1 = x + (n_mine + 3) / 4, quarter2 = x + (2 * n_mine + 3) / 4,
                  quarter3 = x + (3 * n_mine + 3) / 4;
    auto set_prio = [&](int64_t xc) {
      if (xc < quarter1) __builtin_amdgcn_s_setprio(3);
      else if (xc < quarter2) __builtin_amdgcn_s_setprio(2);
      else if (xc < quarter3) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    };
    // list entry y (< T) -> sequence sb (the last with Hkv pref[sb] <= y, which has pages),
    // KV head sg, page sp of its np full pages
    auto locate = [&](int64_t y, int& sb, int& sg, int& sp, int& np) {
      int lo2 = 0, hi2 = batch;
      while (hi2 - lo2 > 1) {
        const int mid = (lo2 + hi2) >> 1;
        if (int64_t(num_kv_heads) * sm.pref[mid] <= y) lo2 = mid; else hi2 = mid;
      }
      sb = __builtin_amdgcn_readfirstlane(lo2);
      np = __builtin_amdgcn_readfirstlane(sm.pref[sb + 1] - sm.pref[sb]);
      const int off = int(y - int64_t(num_kv_heads) * sm.pref[sb]);
      sg = __builtin_amdgcn_readfirstlane(off / np);
      sp = __builtin_amdgcn_readfirstlane(off - sg * np);
    };
    int sb, sg, sp, np;
    locate(x, sb, sg, sp, np);
    uint4 qraw[4];
    q_loads(sb, sg, qraw);
    int64_t cur = rec_of(block_table + int64_t(sb) * bt_stride, sp, np, sg);
    load_meta<AUX, FMT, NG>(t, krec_of(cur), vrec_of(cur), lo);
    load_kcodes<AUX>(t, krec_of(cur), lo);
    load_vcodes<AUX>(t, vrec_of(cur), lo);
    rotate_loaded_q(qraw);   // the first segment's q (later ones: at the end of the previous)
    while (x < x_end) {
      // this segment: pages sp .. sp + n - 1 of (sb, sg)
      const int n = int(min(x_end - x, int64_t(np - sp)));
      const int32_t* bt_r = block_table + int64_t(sb) * bt_stride;
      // the list entry after the segment (its loads are issued by the segment's last page)
      const int64_t x_next = x + n;
      int nb = sb, ng = sg, nsp = 0, nnp = 0;
      int64_t after = -1;
      if (x_next < x_end) {
        locate(x_next, nb, ng, nsp, nnp);
        after = rec_of(block_table + int64_t(nb) * bt_stride, nsp, nnp, ng);
      }
      m_run = -INFINITY;
      l_part = 0.f;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[bb][i] = 0.f;
      for (int k = 0; k < n; ++k) {
        const int64_t next = k + 1 < n ? rec_of(bt_r, sp + k + 1, np, sg) : after;
        set_prio(x + k);
        process(t, next, cur >= 0, kTile);
        cur = next;
      }
      // this wave's partial of the segment, slot wi + (sb Hkv + sg)
      const float l_run = combine_columns();
      if (hi && head_ok) {
        float* part = ws + ((int64_t(wi) + int64_t(sb) * num_kv_heads + sg) * G + h) * kPartStride;
        if (gq == 0) {
          part[0] = m_run;
          part[1] = l_run;
        }
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
          *reinterpret_cast<float4*>(part + 4 + 16 * bb + 4 * gq) =
              make_float4(acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]);
      }
      x = x_next;
      sb = nb;
      sg = ng;
      sp = nsp;
      np = nnp;
      if (x < x_end) {   // the next segment's q, while its first page's loads are in flight
        uint4 qn[4];
        q_loads(sb, sg, qn);
        rotate_loaded_q(qn);
      }
    }
    return;
  } else {
  const int32_t* bt_row = block_table + int64_t(rg.b) * bt_stride;
  const int wslot = __builtin_amdgcn_readfirstlane(slot0 + w);   // this wave's first slot
  uint4 qraw[4];
  q_loads(b, g, qraw);
  int64_t cur = rec_of(bt_row, wslot, n_full, g);
  load_meta<AUX, FMT, NG>(t, krec_of(cur), vrec_of(cur), lo);
  load_kcodes<AUX>(t, krec_of(cur), lo);
  load_vcodes<AUX>(t, vrec_of(cur), lo);
  // q is rotated while the first page's loads are in flight
  rotate_loaded_q(qraw);
  // pages of this wave: slots wslot, wslot + 4, ... below n_full, at most tpw of them
  // (a loop with one exit keeps the running state in place across iterations)
  const int n_here = wslot < n_full ? min(tpw, (n_full - wslot + 3) >> 2) : 0;
  for (int k = 0; k < n_here; ++k) {
    const int64_t next = k + 1 < n_here ? rec_of(bt_row, wslot + 4 * (k + 1), n_full, g) : -1;
    process(t, next, cur >= 0, wslot + 4 * k == n_full - 1 ? rg.mask_lim : kTile);
    cur = next;
  }

  // ---- combine the high / low columns, then the 4 waves --------------------------------
  const float l_run = combine_columns();
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
}

// Merge the splits of one (sequence, query head): log-sum-exp weights, H^T on the page
// part (rotated space), plus the raw-space tail; float16 output. One wave per (query head,
// sequence), four heads per 256-thread workgroup: lane l owns channels l and l + 64, so every
// reduction and the whole H^T stay inside the wave (no workgroup barrier). Split weights are
// computed once into the wave's LDS slot, then every lane streams its two channels of all
// partials (independent loads).
// BAL: the balanced layout of decode_pages_kernel (n_page_wg page workgroups); the partials of
// segment (b, g) are the slots i + (b Hkv + g) of the waves i whose page ranges meet it.
// The split weights live in dynamic LDS, w_cap + 1 floats per head (w_cap >= the splits any
// row uses; the tail's weight at index w_cap): a small read keeps its workgroups small.
template <bool BAL>
__global__ void __launch_bounds__(256)
decode_merge_kernel(int32_t num_q_heads, int32_t num_kv_heads,
                    const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                    const int32_t* __restrict__ cu_q, int32_t batch, int32_t tiles_per_split,
                    int32_t n_splits, int32_t has_tail, const float* __restrict__ ws,
                    int32_t n_page_wg, int32_t w_cap, __half* __restrict__ out) {
  extern __shared__ float merge_w[];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* wsh = merge_w + wv * (w_cap + 1);
  // a head past the last runs along and stores nothing
  const int hq = min(4 * int(blockIdx.x) + wv, num_q_heads - 1);
  const bool head_ok = 4 * int(blockIdx.x) + wv < num_q_heads;
  const int b = blockIdx.y;   // b: output row
  const RowGeom rg = row_geometry(b, seq_lens, max_seq_len, cu_q, batch);
  const bool tail = has_tail && rg.tail_len != 0;
  int used;
  const float* base;     // the first split's partial
  int64_t pstride;       // floats from one split's partial to the next
  const float* tailp;    // the tail partial
  if constexpr (BAL) {
    // full pages before sequence b and in all: the prefix sums the pages kernel stored
    const int32_t* pref = reinterpret_cast<const int32_t*>(
        ws + balanced_pref_offset(n_page_wg, batch, num_q_heads, num_kv_heads));
    const int before = pref[b], total = pref[batch];
    const int G = num_q_heads / num_kv_heads;
    const int g = hq / G, hh = hq - g * G;
    const int P = rg.n_slots;                        // full pages of b
    const int64_t T = int64_t(num_kv_heads) * total;
    const int64_t W = T < 4 * int64_t(n_page_wg) ? T : 4 * int64_t(n_page_wg);
    used = 0;
    base = ws;
    if (P > 0) {
      // wave of list entry y: floor(((y + 1) W - 1) / T)
      const int64_t F0 = int64_t(num_kv_heads) * before + int64_t(g) * P;
      const int64_t i0 = ((F0 + 1) * W - 1) / T, i1 = ((F0 + P) * W - 1) / T;
      used = int(i1 - i0 + 1);
      base = ws + ((i0 + int64_t(b) * num_kv_heads + g) * G + hh) * kPartStride;
    }
    pstride = int64_t(G) * kPartStride;
    tailp = ws + balanced_tail_offset(n_page_wg, batch, num_q_heads, num_kv_heads) +
            (int64_t(b) * num_q_heads + hq) * kPartStride;
  } else {
    used = (rg.n_slots + tiles_per_split - 1) / tiles_per_split;
    base = ws + (int64_t(b) * num_q_heads + hq) * (n_splits + 1) * kPartStride;
    pstride = kPartStride;
    tailp = base + int64_t(n_splits) * kPartStride;
  }
  // 1. global max over the used splits (and the tail); the (m, l) of this lane's first split
  // and of the tail stay in registers for step 2 (one memory round trip fewer)
  float m_first = -INFINITY, l_first = 0.f, m_tail = -INFINITY, l_tail = 0.f;
  if (lane < used) {
    m_first = base[lane * pstride];
    l_first = base[lane * pstride + 1];
  }
  if (tail && lane == 0) {
    m_tail = tailp[0];
    l_tail = tailp[1];
  }
  float M = fmaxf(m_first, m_tail);
  for (int s = lane + 64; s < used; s += 64) M = fmaxf(M, base[s * pstride]);
  for (int off = 32; off >= 1; off >>= 1)
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(M))));
  // 2. split weights exp2(m_s - M) into the wave's LDS slot, and the total l
  float lsum = 0.f;
  for (int s = lane; s < used; s += 64) {
    const float ms = s == lane ? m_first : base[s * pstride];
    const float ls = s == lane ? l_first : base[s * pstride + 1];
    const float e = M == -INFINITY ? 0.f : exp2f(ms - M);
    wsh[s] = e;
    lsum = fmaf(e, ls, lsum);
  }
  if (lane == 0) {
    const float e = (tail && M != -INFINITY) ? exp2f(m_tail - M) : 0.f;
    wsh[w_cap] = e;
    if (tail) lsum = fmaf(e, l_tail, lsum);
  }
  for (int off = 32; off >= 1; off >>= 1)
    lsum += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ off) << 2, __float_as_int(lsum)));
  // the wave's LDS writes land before its reads below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 3. weighted sum of the rotated accumulators, channels lane and lane + 64
  // (16 independent loads in flight per round trip, then 8, 4, 1; the order of the sums
  // does not depend on the unrolling)
  float a0 = 0.f, a1 = 0.f;
  const float* acc0 = base + 4 + lane;
  int s = 0;
  for (; s + 8 <= used; s += 8) {
    float v0[8], v1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v0[k] = acc0[(s + k) * pstride];
      v1[k] = acc0[(s + k) * pstride + 64];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a0 = fmaf(wsh[s + k], v0[k], a0);
      a1 = fmaf(wsh[s + k], v1[k], a1);
    }
  }
  if (s + 4 <= used) {
    float v0[4], v1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v0[k] = acc0[(s + k) * pstride];
      v1[k] = acc0[(s + k) * pstride + 64];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a0 = fmaf(wsh[s + k], v0[k], a0);
      a1 = fmaf(wsh[s + k], v1[k], a1);
    }
    s += 4;
  }
  for (; s < used; ++s) {
    a0 = fmaf(wsh[s], acc0[s * pstride], a0);
    a1 = fmaf(wsh[s], acc0[s * pstride + 64], a1);
  }
  // 4. H^T = H over the 128 channels: bits 0..5 across the lanes, bit 6 within the lane
  {
#define KVARN_MSTAGE(M_, FN)                          \
    {                                                 \
      const float p0 = FN(a0), p1 = FN(a1);           \
      a0 = (lane & (M_)) ? (p0 - a0) : (a0 + p0);     \
      a1 = (lane & (M_)) ? (p1 - a1) : (a1 + p1);     \
    }
    KVARN_MSTAGE(1, dpp_f<kDppQuadXor1>)
    KVARN_MSTAGE(2, dpp_f<kDppQuadXor2>)
    KVARN_MSTAGE(4, swz_xor_f<4>)
    KVARN_MSTAGE(8, dpp_f<kDppRowRor8>)
    KVARN_MSTAGE(16, swz_xor_f<16>)
    KVARN_MSTAGE(32, shfl_xor32_f)
#undef KVARN_MSTAGE
    const float lo = a0 + a1, hi = a0 - a1;
    a0 = lo * kInvSqrt128;
    a1 = hi * kInvSqrt128;
  }
  if (tail) {
    a0 = fmaf(wsh[w_cap], tailp[4 + lane], a0);
    a1 = fmaf(wsh[w_cap], tailp[4 + 64 + lane], a1);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (head_ok) {
    __half* o = out + (int64_t(b) * num_q_heads + hq) * kDim;
    o[lane] = __float2half_rn(a0 * inv);
    o[lane + 64] = __float2half_rn(a1 * inv);
  }
}

}  // namespace

int32_t decode_tiles_per_wave(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t max_full = max_seq_len / kTile;
  const int64_t work = int64_t(batch) * num_kv_heads * max_full;
  // 1,024 waves, half a round of the resident ones (one per SIMD): on one 128K-token sequence
  // 8 pages per wave beat 4 pages on twice the waves (35-37 against 38-41 us, A/B in one run)
  int64_t tpw = (work + 1023) / 1024;
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

// Page workgroups of the balanced layout for a decode of this shape (one query row per
// sequence), or 0 where the split layout runs: a single sequence (its splits are already
// even), more sequences than the LDS prefix holds, or a page list that could reach 2^31.
int32_t decode_balanced_wg(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t max_full = max_seq_len / kTile;
  const int64_t work = int64_t(batch) * num_kv_heads * max_full;   // >= the page list length
  if (batch < 2 || batch > kMaxBalancedRows || max_full < 1 || work >= (int64_t(1) << 31)) return 0;
  const int64_t wg = (work + 3) / 4;
  return int32_t(wg < kBalancedPageWg ? wg : kBalancedPageWg);
}

// Fixed device scratch of the entry point that allocates nothing (callers that cannot call
// hipMalloc: graph capture, tight serving loops). Each GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` names a host-side stand-in, never a
// device address: kernels get the address decode_scratch() obtained for the current device.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current: the address of this device's copy
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_seq_len) {
  const int32_t ns = decode_num_splits(batch, num_kv_heads, max_seq_len);
  const size_t split = size_t(batch) * num_q_heads * (ns + 1) * kPartStride * sizeof(float);
  const int32_t wg = decode_balanced_wg(batch, num_kv_heads, max_seq_len);
  if (wg == 0) return split;
  const size_t bal = size_t(balanced_pref_offset(wg, batch, num_q_heads, num_kv_heads) + batch + 1) *
                    sizeof(float);
  return bal > split ? bal : split;
}

hipError_t launch_decode(int k_bits, int v_bits, int fmt, int group, const void* q, int32_t rows,
                         int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                         const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                         const int32_t* cu_q, int32_t batch, const void* k_tail,
                         const void* v_tail, float softmax_scale, void* workspace, void* out,
                         hipStream_t stream) {
  // several query rows of one sequence (more rows than sequences): the multi-query kernel
  const bool multi_row = cu_q != nullptr && rows > batch;
  const bool has_tail = k_tail != nullptr && v_tail != nullptr;
  const float qscale = softmax_scale * kLog2e;
  float* ws = static_cast<float*>(workspace);
  // a decode of several sequences: the balanced layout (equal page counts per wave)
  const int32_t bal_wg = cu_q == nullptr ? decode_balanced_wg(rows, num_kv_heads, max_seq_len) : 0;
  if (bal_wg > 0) {
    const int32_t n_wg = bal_wg + (has_tail ? rows * num_kv_heads : 0);
    const hipError_t e = with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
      constexpr int KB = decltype(kb)::value, VB = decltype(vb)::value, FM = decltype(fm)::value,
                    NG = decltype(ng)::value;
      hipLaunchKernelGGL((decode_pages_kernel<KB, VB, FM, NG, kStreamLoad, true>), dim3(n_wg),
                         dim3(kThreads), 0, stream, static_cast<const __half*>(q), num_q_heads,
                         num_kv_heads, static_cast<const uint8_t*>(k_pool),
                         static_cast<const uint8_t*>(v_pool), pool_num_pages, block_table,
                         bt_stride, seq_lens, max_seq_len, cu_q, batch, qscale * kInvSqrt128,
                         1, 1, 0, static_cast<const __half*>(k_tail),
                         static_cast<const __half*>(v_tail), qscale, ws, bal_wg);
    });
    if (e != hipSuccess) return e;
    // a segment's partials come from at most all 4 bal_wg waves
    const int32_t cap = 4 * bal_wg;
    hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((num_q_heads + 3) / 4, rows), dim3(256),
                       4 * (cap + 1) * sizeof(float), stream, num_q_heads, num_kv_heads, seq_lens,
                       max_seq_len, cu_q, batch, 1, 1, has_tail ? 1 : 0,
                       static_cast<const float*>(ws), bal_wg, cap, static_cast<__half*>(out));
    return hipGetLastError();
  }
  const int32_t tpw = decode_tiles_per_wave(rows, num_kv_heads, max_seq_len);
  const int32_t per_split =
      multi_row ? mq_slots_per_split(rows, num_q_heads, num_kv_heads, max_seq_len) : 4 * tpw;
  const int32_t ns = multi_row ? mq_num_splits(rows, num_q_heads, num_kv_heads, max_seq_len)
                               : decode_num_splits(rows, num_kv_heads, max_seq_len);
  // page splits (only if a full page can exist) plus, with tail buffers, one tail split
  const int32_t n_split_wg = (max_seq_len >= kTile ? ns : 0) + (has_tail ? 1 : 0);
  if (n_split_wg > 0) {
    // without pages the only split launched is the tail, which must land on index ns
    const int32_t first = max_seq_len >= kTile ? 0 : ns;
    // (KV head, row) fastest, splits slowest: workgroups are dealt to the 8 XCDs round-robin
    // in linear order, so consecutive ones must all carry work (a split axis of period 2,
    // pages + tail, would leave every page workgroup on the even XCDs)
    hipError_t e;
    if (multi_row) {
      e = launch_mq_pages(k_bits, v_bits, fmt, group, q, rows, num_q_heads, num_kv_heads, k_pool, v_pool,
                          pool_num_pages, block_table, bt_stride, seq_lens, max_seq_len, cu_q,
                          batch, k_tail, v_tail, qscale * kInvSqrt128, qscale, per_split, ns,
                          n_split_wg, first, workspace, stream);
    } else {
      e = with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
        constexpr int KB = decltype(kb)::value, VB = decltype(vb)::value, FM = decltype(fm)::value,
                    NG = decltype(ng)::value;
        // decode streams every page once; a read with one query per sequence reuses them
        auto kernel = cu_q ? decode_pages_kernel<KB, VB, FM, NG, kReuseLoad, false>
                           : decode_pages_kernel<KB, VB, FM, NG, kStreamLoad, false>;
        hipLaunchKernelGGL(kernel, dim3(rows * num_kv_heads, n_split_wg), dim3(kThreads), 0,
                           stream, static_cast<const __half*>(q), num_q_heads, num_kv_heads,
                           static_cast<const uint8_t*>(k_pool),
                           static_cast<const uint8_t*>(v_pool), pool_num_pages, block_table,
                           bt_stride, seq_lens, max_seq_len, cu_q, batch, qscale * kInvSqrt128,
                           tpw, ns, first, static_cast<const __half*>(k_tail),
                           static_cast<const __half*>(v_tail), qscale, ws, 0);
      });
    }
    if (e != hipSuccess) return e;
  }
  // every row uses at most ns splits (ns <= kMaxMergeSplits by the split sizing)
  hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((num_q_heads + 3) / 4, rows), dim3(256),
                     4 * (ns + 1) * sizeof(float), stream, num_q_heads, num_kv_heads, seq_lens,
                     max_seq_len, cu_q, batch, per_split, ns, has_tail ? 1 : 0,
                     static_cast<const float*>(ws), 0, ns, static_cast<__half*>(out));
  return hipGetLastError();
}

}  // namespace kvarn

// KVarN multi-query read for gfx950: causal attention of many query rows per sequence over
// the quantized pages (the read path of a prefill chunk), 16 query vectors per wave.
#include "decode_common.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

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

template <int NG>
struct MqSmem {
  WaveMeta<NG> meta[4];
  union {
    float4 q[4][8][64];   // q_rot per wave: [k][lane] = channels 32 gq + 4k .. 4k + 3
    TailSmem tail;        // tail split: the staged-token attention
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

template <int KB, int VB, int FMT, int NG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mq_pages_kernel(const __half* __restrict__ q, int32_t num_q_heads, int32_t num_kv_heads,
                const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                int64_t pool_num_pages, const int32_t* __restrict__ block_table,
                int32_t bt_stride, const int32_t* __restrict__ seq_lens, int32_t max_seq_len,
                const int32_t* __restrict__ cu_q, int32_t batch, int32_t n_rows, float qscale,
                int32_t slots_per_split, int32_t n_splits, int32_t split_base,
                const __half* __restrict__ k_tail, const __half* __restrict__ v_tail,
                float tail_qscale, float* __restrict__ ws) {
  __shared__ MqSmem<NG> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int split = split_base + blockIdx.z, g = blockIdx.y;
  const int G = num_q_heads / num_kv_heads;
  const int R = 16 / G;                                   // rows per wave
  const MqWindow win = mq_window(blockIdx.x, 4 * R, cu_q, batch, n_rows);
  if (split == n_splits) {   // the tails of the window's rows, one row after the other
    for (int row = win.r0; row < win.r1; ++row) {   // uniform over the workgroup
      const RowGeom rgr = row_geometry(row, seq_lens, max_seq_len, cu_q, batch);
      tail_partial(q, num_q_heads, num_kv_heads, k_tail, v_tail, row, rgr.b, g, rgr.tail_len,
                   tail_qscale, n_splits, ws, sm.tail);
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

  WaveMeta<NG>& wm = sm.meta[w];
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
    return record_rsrc(uniform_ptr(k_pool + uint64_t(r) * uint32_t(key_record<KB, FMT, NG>())),
                       page < 0 ? 0 : key_record<KB, FMT, NG>());
  };
  auto vrec_of = [&](int64_t page) {
    const uint32_t ps = __builtin_amdgcn_readfirstlane(uint32_t(page < 0 ? 0 : page));
    const uint32_t r = ps * uint32_t(num_kv_heads) + uint32_t(g);
    return record_rsrc(uniform_ptr(v_pool + uint64_t(r) * uint32_t(val_record<VB, FMT, NG>())),
                       page < 0 ? 0 : val_record<VB, FMT, NG>());
  };

  PageRegs<KB, VB> t;
  int64_t cur = page_of(s0);
  load_meta<kReuseLoad, FMT, NG>(t, krec_of(cur), vrec_of(cur), lo);
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
    page_factors<FMT, NG>(t, wm, l, maxq, fk, fv);
    load_meta<kReuseLoad, FMT, NG>(t, krec_of(next), vrec_of(next), lo);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- QK per key group (NG = 2: token blocks 0..3 take the factors of tokens 0..63,
    // blocks 4..7 those of 64..127): B operand q_rot * ka (high, low), bias = q_rot . kb;
    // C rows = tokens 16 tb + 4 gq + i, column = this lane's query
    float sc[8][4];
#pragma unroll
    for (int hq = 0; hq < NG; ++hq) {
      H8 bqh[4], bql[4];
      float bias;
      {
        float bpart = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float4 ka0 = wm.ka[hq][8 * gq + 2 * s], ka1 = wm.ka[hq][8 * gq + 2 * s + 1];
          const float4 kb0 = wm.kb[hq][8 * gq + 2 * s], kb1 = wm.kb[hq][8 * gq + 2 * s + 1];
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
      const float4v binit = {bias, bias, bias, bias};
      const float* kt = reinterpret_cast<const float*>(wm.kt);
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
    // B operand of PV for value group hv (the softmax weights times the group's value
    // factors, high / low) and its zero-point correction. NG = 1 turns the scores into
    // weights here, adding them to psum; NG = 2 reads weights computed beforehand.
    auto pv_operands = [&](int hv, H8 (&bph)[4], H8 (&bpl)[4], float& psum) -> float {
      float zpart = 0.f;
      const float* vp = reinterpret_cast<const float*>(wm.vp[hv]);
      const float* vz = reinterpret_cast<const float*>(wm.vz[hv]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tb = 2 * s + e;
          const float4 vp4 = *reinterpret_cast<const float4*>(vp + 16 * tb + 4 * gq);
          const float4 vz4 = *reinterpret_cast<const float4*>(vz + 16 * tb + 4 * gq);
          float p0 = sc[tb][0], p1 = sc[tb][1], p2 = sc[tb][2], p3 = sc[tb][3];
          if constexpr (NG == 1) {
            p0 = exp2_fast(p0 - m_sub);
            p1 = exp2_fast(p1 - m_sub);
            p2 = exp2_fast(p2 - m_sub);
            p3 = exp2_fast(p3 - m_sub);
            psum += (p0 + p1) + (p2 + p3);
          }
          zpart = fmaf(p0, vz4.x, fmaf(p1, vz4.y, fmaf(p2, vz4.z, fmaf(p3, vz4.w, zpart))));
          split_pk(p0 * vp4.x, p1 * vp4.y, bph[s].u[2 * e], bpl[s].u[2 * e]);
          split_pk(p2 * vp4.z, p3 * vp4.w, bph[s].u[2 * e + 1], bpl[s].u[2 * e + 1]);
        }
      }
      return rows4_sum(zpart);
    };
    // PV of channel blocks bb0 .. bb0 + 8 / NG - 1 (one value group); C rows = channels
    // 16 bb + 4 gq + i
    auto pv_blocks = [&](const H8 (&bph)[4], const H8 (&bpl)[4], float vcorr, int bb0) {
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
    };
    auto rescale = [&]() {
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[bb][i] *= alpha;
      }
    };
    // ---- softmax weights and PV (NG = 2: channel blocks 0..3 take the value factors of
    // channels 0..63, blocks 4..7 those of channels 64..127) --------------------------------
    if constexpr (NG == 1) {
      H8 bph[4], bpl[4];
      float psum = 0.f;
      const float vcorr = pv_operands(0, bph, bpl, psum);
      l_part = fmaf(l_part, alpha, psum);
      m_run = m_new;
      rescale();
      pv_blocks(bph, bpl, vcorr, 0);
    } else {
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tb][i] = exp2_fast(sc[tb][i] - m_sub);
        psum += (sc[tb][0] + sc[tb][1]) + (sc[tb][2] + sc[tb][3]);
      }
      l_part = fmaf(l_part, alpha, psum);
      m_run = m_new;
      rescale();
#pragma unroll
      for (int hv = 0; hv < NG; ++hv) {
        H8 bph[4], bpl[4];
        const float vcorr = pv_operands(hv, bph, bpl, psum);
        pv_blocks(bph, bpl, vcorr, 8 / NG * hv);
      }
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

}  // namespace

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

hipError_t launch_mq_pages(int k_bits, int v_bits, int fmt, int group, const void* q, int32_t rows,
                          int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                          const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                          int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                          const int32_t* cu_q, int32_t batch, const void* k_tail,
                          const void* v_tail, float qscale_pages, float qscale_tail,
                          int32_t slots_per_split, int32_t n_splits, int32_t n_split_wg,
                          int32_t split_base, void* workspace, hipStream_t stream) {
  // 16 query vectors per wave, windows of 4R rows per workgroup
  const int R = 16 / (num_q_heads / num_kv_heads);
  return with_preset(k_bits, v_bits, fmt, group, [&](auto kb, auto vb, auto fm, auto ng) {
    constexpr int KB = decltype(kb)::value, VB = decltype(vb)::value, FM = decltype(fm)::value,
                    NG = decltype(ng)::value;
    hipLaunchKernelGGL((mq_pages_kernel<KB, VB, FM, NG>),
                       dim3((rows + 4 * R - 1) / (4 * R) + batch, num_kv_heads, n_split_wg),
                       dim3(kThreads), 0, stream, static_cast<const __half*>(q), num_q_heads,
                       num_kv_heads, static_cast<const uint8_t*>(k_pool),
                       static_cast<const uint8_t*>(v_pool), pool_num_pages, block_table,
                       bt_stride, seq_lens, max_seq_len, cu_q, batch, rows, qscale_pages,
                       slots_per_split, n_splits, split_base, static_cast<const __half*>(k_tail),
                       static_cast<const __half*>(v_tail), qscale_tail,
                       static_cast<float*>(workspace));
  });
}

}  // namespace kvarn

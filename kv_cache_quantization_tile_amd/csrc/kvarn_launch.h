// Internal launchers of the KVarN HIP kernels (called by the C ABI after validation).
// k_bits / v_bits: key and value code widths of the preset (4/2: kvarn_k4v2_g*,
// 2/2: kvarn_k2v2_g*, 4/4: kvarn_k4v4_g*); fmt: record format (1 separate metadata,
// 2 folded); group: 128 or 64 elements per quantization group.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace kvarn {

// Calls f(kb, vb, fm, ng) with the preset's code widths, the record format and the groups
// per key channel / value token (1: group 128, 2: group 64) as std::integral_constant<int, ...>
// values (one kernel instantiation per preset, format and group size), then returns the
// launch status; hipErrorInvalidValue for a pair that is no preset, a format other than 1 and
// 2, or a group size other than 128 and 64.
template <typename F>
hipError_t with_preset(int k_bits, int v_bits, int fmt, int group, F&& f) {
  using B2 = std::integral_constant<int, 2>;
  using B4 = std::integral_constant<int, 4>;
  using F1 = std::integral_constant<int, 1>;
  using F2 = std::integral_constant<int, 2>;
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  auto by_group = [&](auto kb, auto vb, auto fm) {
    if (group == 128) f(kb, vb, fm, G1{});
    else f(kb, vb, fm, G2{});
  };
  auto by_format = [&](auto kb, auto vb) {
    if (fmt == 1) by_group(kb, vb, F1{});
    else by_group(kb, vb, F2{});
  };
  if (fmt != 1 && fmt != 2) return hipErrorInvalidValue;
  if (group != 128 && group != 64) return hipErrorInvalidValue;
  if (k_bits == 4 && v_bits == 2)
    by_format(B4{}, B2{});
  else if (k_bits == 2 && v_bits == 2)
    by_format(B2{}, B2{});
  else if (k_bits == 4 && v_bits == 4)
    by_format(B4{}, B4{});
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_tiles(int kind, int k_bits, int v_bits, int fmt, int group, const void* src,
                                 int64_t token_stride, int64_t head_stride, int64_t src_num_tokens,
                                 const int64_t* tile_src_token, const int32_t* tile_dst_page,
                                 int32_t n_tiles, int32_t num_kv_heads, void* pool,
                                 int64_t pool_num_pages, int n_iters, hipStream_t stream);

hipError_t launch_quantize_kv(int k_bits, int v_bits, int fmt, int group, const void* k_src, const void* v_src,
                              int64_t token_stride, int64_t head_stride, int64_t src_num_tokens,
                              const int64_t* tile_src_token, const int32_t* tile_dst_page,
                              int32_t n_tiles, int32_t num_kv_heads, void* k_pool, void* v_pool,
                              int64_t pool_num_pages, int n_iters, hipStream_t stream);

hipError_t launch_dequantize_tiles(int kind, int k_bits, int v_bits, int fmt, int group, const void* pool,
                                   int64_t pool_num_pages, const int32_t* pages, int32_t n_tiles,
                                   int32_t num_kv_heads, void* dst, hipStream_t stream);

hipError_t launch_write_tokens(int k_bits, int v_bits, int fmt, int group, const void* k_new, const void* v_new,
                               int32_t total_new, const int32_t* cu_new, int32_t max_new,
                               int32_t batch, int32_t num_kv_heads, const int32_t* seq_lens,
                               void* k_tail, void* v_tail, const int32_t* block_table,
                               int32_t bt_stride, void* k_pool, void* v_pool,
                               int64_t pool_num_pages, int n_iters, hipStream_t stream);

hipError_t launch_append_tokens(int k_bits, int v_bits, int fmt, int group, const void* k_new, const void* v_new,
                                int32_t batch, int32_t num_kv_heads, const int32_t* seq_lens,
                                void* k_tail, void* v_tail, const int32_t* block_table,
                                int32_t bt_stride, void* k_pool, void* v_pool,
                                int64_t pool_num_pages, int n_iters, hipStream_t stream);

// Bytes of the fixed device scratch that kvarn_decode_attention_noalloc uses as its
// workspace, and the address of the current device's copy (taken once per device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

int32_t decode_tiles_per_wave(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len);
int32_t decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len);
size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_seq_len);
// multi-query read (several query rows per sequence): page slots per split, splits, and the
// workspace a chunk read needs (either layout)
int32_t mq_slots_per_split(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t max_seq_len);
int32_t mq_num_splits(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t max_seq_len);
size_t chunk_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t max_seq_len);

// The page splits (and tail split) of a multi-query read: n_split_wg splits from split_base;
// partials into workspace for the merge that launch_decode runs next. qscale_pages includes
// the 1/sqrt(128) of the query rotation; both scales include log2(e).
hipError_t launch_mq_pages(int k_bits, int v_bits, int fmt, int group, const void* q, int32_t rows,
                          int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                          const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                          int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                          const int32_t* cu_q, int32_t batch, const void* k_tail,
                          const void* v_tail, float qscale_pages, float qscale_tail,
                          int32_t slots_per_split, int32_t n_splits, int32_t n_split_wg,
                          int32_t split_base, void* workspace, hipStream_t stream);

// rows output rows; cu_q == nullptr: row b is sequence b (decode, rows == batch), else the
// query rows of sequence b are cu_q[b] .. cu_q[b+1]-1 (the last positions of its cache)
hipError_t launch_decode(int k_bits, int v_bits, int fmt, int group, const void* q, int32_t rows,
                         int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                         const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                         const int32_t* cu_q, int32_t batch, const void* k_tail,
                         const void* v_tail, float softmax_scale, void* workspace, void* out,
                         hipStream_t stream);

}  // namespace kvarn

// C ABI of the KVarN library: host-side validation, then kernel launches.
// Every check runs before anything is enqueued; see include/kvarn.h for the contract.
#include <math.h>
#include <string.h>

#include "../../include/kvarn.h"
#include "kvarn_launch.h"

namespace {

constexpr int32_t kMaxIters = 64;
constexpr int32_t kMaxGroup = 8;  // query heads per KV head handled by one decode wave

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvarn_status launch_status(hipError_t e) { return e == hipSuccess ? KVARN_OK : KVARN_ERR_HIP; }

// Parse a non-negative decimal integer at *p (advancing it); -1 if none or too large.
int parse_uint(const char** p) {
  const char* s = *p;
  if (*s < '0' || *s > '9') return -1;
  long v = 0;
  while (*s >= '0' && *s <= '9') {
    v = v * 10 + (*s - '0');
    if (v > 1000000) return -1;
    ++s;
  }
  *p = s;
  return int(v);
}

}  // namespace

extern "C" {

int32_t kvarn_abi_version(void) { return KVARN_ABI_VERSION; }
int32_t kvarn_format_version(void) { return KVARN_FORMAT_VERSION; }

const char* kvarn_status_str(kvarn_status status) {
  switch (status) {
    case KVARN_OK: return "ok";
    case KVARN_ERR_INVALID_ARG: return "invalid argument";
    case KVARN_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVARN_ERR_WORKSPACE: return "workspace too small";
    case KVARN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

kvarn_status kvarn_params_check(const kvarn_params* p) {
  if (!p) return KVARN_ERR_INVALID_ARG;
  if (p->head_dim <= 0 || p->tile_tokens <= 0 || p->group <= 0 || p->k_bits <= 0 ||
      p->v_bits <= 0 || p->sinkhorn_iters < 0 || p->sinkhorn_iters > kMaxIters)
    return KVARN_ERR_INVALID_ARG;
  if (p->format != KVARN_FORMAT_SEPARATE && p->format != KVARN_FORMAT_FOLDED)
    return KVARN_ERR_INVALID_ARG;
  // presets kvarn_k4v2_g128 (released), kvarn_k2v2_g128 and kvarn_k4v4_g128, each also with
  // group 64 (_g64)
  const bool preset = (p->k_bits == 4 && p->v_bits == 2) || (p->k_bits == 2 && p->v_bits == 2) ||
                      (p->k_bits == 4 && p->v_bits == 4);
  if (p->head_dim != 128 || p->tile_tokens != 128 || (p->group != 128 && p->group != 64) ||
      !preset)
    return KVARN_ERR_UNSUPPORTED;
  return KVARN_OK;
}

kvarn_status kvarn_params_from_dtype(const char* dtype, int32_t sinkhorn_iters, kvarn_params* out) {
  if (!dtype || !out) return KVARN_ERR_INVALID_ARG;
  const char* s = dtype;
  if (strncmp(s, "kvarn_k", 7) != 0) return KVARN_ERR_INVALID_ARG;
  s += 7;
  const int kb = parse_uint(&s);
  if (kb < 0 || *s != 'v') return KVARN_ERR_INVALID_ARG;
  ++s;
  const int vb = parse_uint(&s);
  if (vb < 0 || strncmp(s, "_g", 2) != 0) return KVARN_ERR_INVALID_ARG;
  s += 2;
  const int grp = parse_uint(&s);
  if (grp < 0 || *s != '\0') return KVARN_ERR_INVALID_ARG;
  kvarn_params p;
  p.head_dim = 128;
  p.tile_tokens = 128;
  p.k_bits = kb;
  p.v_bits = vb;
  p.group = grp;
  p.sinkhorn_iters = sinkhorn_iters;
  p.format = KVARN_FORMAT_SEPARATE;
  if (kb == 0 || vb == 0 || grp == 0) return KVARN_ERR_INVALID_ARG;
  const kvarn_status st = kvarn_params_check(&p);
  if (st != KVARN_OK) return st;
  *out = p;
  return KVARN_OK;
}

size_t kvarn_page_bytes(const kvarn_params* p, kvarn_kind kind) {
  if (kvarn_params_check(p) != KVARN_OK) return 0;
  // codes, then float16 vectors of 128: the normalizers (2 separate, 1 folded), then one
  // scale and one zero vector per group of a key channel / value token (1 for group 128, 2
  // for group 64)
  const size_t meta = 256 * ((p->format == KVARN_FORMAT_SEPARATE ? 2 : 1) + 2 * (128 / p->group));
  if (kind == KVARN_K) return (p->k_bits == 4 ? 8192 : 4096) + meta;
  if (kind == KVARN_V) return (p->v_bits == 4 ? 8192 : 4096) + meta;
  return 0;
}

kvarn_status kvarn_quantize_tiles(const kvarn_params* params, kvarn_kind kind, const void* src,
                                  int64_t src_token_stride, int64_t src_head_stride,
                                  int64_t src_num_tokens, const int64_t* tile_src_token,
                                  const int32_t* tile_dst_page, int32_t n_tiles,
                                  int32_t num_kv_heads, void* pool, int64_t pool_num_pages,
                                  void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (kind != KVARN_K && kind != KVARN_V) return KVARN_ERR_INVALID_ARG;
  if (n_tiles < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 || src_num_tokens < 0 ||
      pool_num_pages < 0 || src_token_stride < 0 || src_head_stride < 0)
    return KVARN_ERR_INVALID_ARG;
  if (n_tiles == 0) return KVARN_OK;
  if (!src || !tile_src_token || !tile_dst_page || !pool) return KVARN_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(pool) || (src_token_stride % 8) != 0 ||
      (src_head_stride % 8) != 0)
    return KVARN_ERR_INVALID_ARG;
  return launch_status(kvarn::launch_quantize_tiles(
      int(kind), params->k_bits, params->v_bits, params->format, params->group, src, src_token_stride, src_head_stride, src_num_tokens, tile_src_token,
      tile_dst_page, n_tiles, num_kv_heads, pool, pool_num_pages, params->sinkhorn_iters,
      static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_quantize_kv_tiles(const kvarn_params* params, const void* k_src,
                                     const void* v_src, int64_t src_token_stride,
                                     int64_t src_head_stride, int64_t src_num_tokens,
                                     const int64_t* tile_src_token, const int32_t* tile_dst_page,
                                     int32_t n_tiles, int32_t num_kv_heads, void* k_pool,
                                     void* v_pool, int64_t pool_num_pages, void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (n_tiles < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 || src_num_tokens < 0 ||
      pool_num_pages < 0 || src_token_stride < 0 || src_head_stride < 0)
    return KVARN_ERR_INVALID_ARG;
  if (n_tiles == 0) return KVARN_OK;
  if (!k_src || !v_src || !tile_src_token || !tile_dst_page || !k_pool || !v_pool)
    return KVARN_ERR_INVALID_ARG;
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_pool) || !aligned16(v_pool) ||
      (src_token_stride % 8) != 0 || (src_head_stride % 8) != 0)
    return KVARN_ERR_INVALID_ARG;
  return launch_status(kvarn::launch_quantize_kv(
      params->k_bits, params->v_bits, params->format, params->group,
      k_src, v_src, src_token_stride, src_head_stride, src_num_tokens, tile_src_token,
      tile_dst_page, n_tiles, num_kv_heads, k_pool, v_pool, pool_num_pages,
      params->sinkhorn_iters, static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_dequantize_tiles(const kvarn_params* params, kvarn_kind kind, const void* pool,
                                    int64_t pool_num_pages, const int32_t* pages, int32_t n_tiles,
                                    int32_t num_kv_heads, void* dst, void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (kind != KVARN_K && kind != KVARN_V) return KVARN_ERR_INVALID_ARG;
  if (n_tiles < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 || pool_num_pages < 0)
    return KVARN_ERR_INVALID_ARG;
  if (n_tiles == 0) return KVARN_OK;
  if (!pool || !pages || !dst) return KVARN_ERR_INVALID_ARG;
  if (!aligned16(pool) || !aligned16(dst)) return KVARN_ERR_INVALID_ARG;
  return launch_status(kvarn::launch_dequantize_tiles(int(kind), params->k_bits, params->v_bits, params->format, params->group, pool, pool_num_pages, pages,
                                                      n_tiles, num_kv_heads, dst,
                                                      static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_append_tokens(const kvarn_params* params, const void* k_new, const void* v_new,
                                 int32_t batch, int32_t num_kv_heads, const int32_t* seq_lens,
                                 void* k_tail, void* v_tail, const int32_t* block_table,
                                 int32_t block_table_stride, void* k_pool, void* v_pool,
                                 int64_t pool_num_pages, void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (batch < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 || block_table_stride <= 0 ||
      pool_num_pages < 0)
    return KVARN_ERR_INVALID_ARG;
  if (batch == 0) return KVARN_OK;
  if (!k_new || !v_new || !seq_lens || !k_tail || !v_tail || !block_table || !k_pool || !v_pool)
    return KVARN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_tail) || !aligned16(v_tail) ||
      !aligned16(k_pool) || !aligned16(v_pool))
    return KVARN_ERR_INVALID_ARG;
  return launch_status(kvarn::launch_append_tokens(
      params->k_bits, params->v_bits, params->format, params->group,
      k_new, v_new, batch, num_kv_heads, seq_lens, k_tail, v_tail, block_table,
      block_table_stride, k_pool, v_pool, pool_num_pages, params->sinkhorn_iters,
      static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_write_tokens(const kvarn_params* params, const void* k_new, const void* v_new,
                                int32_t total_new_tokens, const int32_t* cu_new,
                                int32_t max_new_tokens, int32_t batch,
                                int32_t num_kv_heads, const int32_t* seq_lens, void* k_tail,
                                void* v_tail, const int32_t* block_table,
                                int32_t block_table_stride, void* k_pool, void* v_pool,
                                int64_t pool_num_pages, void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (batch < 0 || batch > 65535 || num_kv_heads <= 0 || num_kv_heads > 32767 ||
      block_table_stride <= 0 || pool_num_pages < 0 || max_new_tokens < 0 ||
      total_new_tokens < 0)
    return KVARN_ERR_INVALID_ARG;
  if (batch == 0 || max_new_tokens == 0 || total_new_tokens == 0) return KVARN_OK;
  if (!k_new || !v_new || !cu_new || !seq_lens || !k_tail || !v_tail || !block_table || !k_pool ||
      !v_pool)
    return KVARN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_tail) || !aligned16(v_tail) ||
      !aligned16(k_pool) || !aligned16(v_pool))
    return KVARN_ERR_INVALID_ARG;
  return launch_status(kvarn::launch_write_tokens(
      params->k_bits, params->v_bits, params->format, params->group,
      k_new, v_new, total_new_tokens, cu_new, max_new_tokens, batch, num_kv_heads, seq_lens, k_tail, v_tail,
      block_table, block_table_stride, k_pool, v_pool, pool_num_pages, params->sinkhorn_iters,
      static_cast<hipStream_t>(stream)));
}

size_t kvarn_decode_workspace_bytes(const kvarn_params* params, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_seq_len) {
  if (kvarn_params_check(params) != KVARN_OK) return 0;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > kMaxGroup)
    return 0;
  return kvarn::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len);
}

size_t kvarn_chunk_workspace_bytes(const kvarn_params* params, int32_t total_q,
                                   int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_seq_len) {
  if (kvarn_params_check(params) != KVARN_OK) return 0;
  if (total_q <= 0 || total_q > 65535 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_seq_len < 0 || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > kMaxGroup)
    return 0;
  return kvarn::chunk_workspace_bytes(total_q, num_q_heads, num_kv_heads, max_seq_len);
}

int32_t kvarn_decode_num_splits(const kvarn_params* params, int32_t batch, int32_t num_kv_heads,
                                int32_t max_seq_len) {
  if (kvarn_params_check(params) != KVARN_OK) return 0;
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return 0;
  return kvarn::decode_num_splits(batch, num_kv_heads, max_seq_len);
}

}  // extern "C"

namespace {

// Every check of kvarn_decode_attention except the workspace size.
kvarn_status check_decode(const kvarn_params* params, const void* q, int32_t batch,
                          int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                          const void* v_pool, int64_t pool_num_pages, const int32_t* block_table,
                          int32_t block_table_stride, const int32_t* seq_lens,
                          int32_t max_seq_len, const void* k_tail, const void* v_tail,
                          float softmax_scale, const void* out) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      pool_num_pages < 0 || block_table_stride < 0 || num_q_heads > 65535 || num_kv_heads > 65535)
    return KVARN_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return KVARN_ERR_INVALID_ARG;
  if (num_q_heads / num_kv_heads > kMaxGroup) return KVARN_ERR_UNSUPPORTED;
  // grid limits: one merge grid row per sequence, one pages workgroup column per
  // (sequence, KV head)
  if (batch > 65535 || int64_t(batch) * num_kv_heads > INT32_MAX) return KVARN_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale)) return KVARN_ERR_INVALID_ARG;
  if (batch == 0) return KVARN_OK;
  if (!q || !seq_lens || !out) return KVARN_ERR_INVALID_ARG;
  if ((k_tail == nullptr) != (v_tail == nullptr)) return KVARN_ERR_INVALID_ARG;
  if (max_seq_len >= 128) {
    if (!k_pool || !v_pool || !block_table) return KVARN_ERR_INVALID_ARG;
    // page records are addressed by a 32-bit index page * num_kv_heads + head
    if (pool_num_pages * int64_t(num_kv_heads) > (int64_t(1) << 32)) return KVARN_ERR_UNSUPPORTED;
    if (block_table_stride < max_seq_len / 128) return KVARN_ERR_INVALID_ARG;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return KVARN_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(out)) return KVARN_ERR_INVALID_ARG;
  if (k_tail && (!aligned16(k_tail) || !aligned16(v_tail))) return KVARN_ERR_INVALID_ARG;
  return KVARN_OK;
}

}  // namespace

extern "C" {

kvarn_status kvarn_decode_attention(const kvarn_params* params, const void* q, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, const void* k_pool,
                                    const void* v_pool, int64_t pool_num_pages,
                                    const int32_t* block_table, int32_t block_table_stride,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    const void* k_tail, const void* v_tail, float softmax_scale,
                                    void* workspace, size_t workspace_bytes, void* out,
                                    void* stream) {
  const kvarn_status st =
      check_decode(params, q, batch, num_q_heads, num_kv_heads, k_pool, v_pool, pool_num_pages,
                   block_table, block_table_stride, seq_lens, max_seq_len, k_tail, v_tail,
                   softmax_scale, out);
  if (st != KVARN_OK || batch == 0) return st;
  if (!workspace) return KVARN_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return KVARN_ERR_INVALID_ARG;
  if (workspace_bytes < kvarn::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len))
    return KVARN_ERR_WORKSPACE;
  return launch_status(kvarn::launch_decode(
      params->k_bits, params->v_bits, params->format, params->group, q, batch, num_q_heads, num_kv_heads, k_pool, v_pool, pool_num_pages, block_table,
      block_table_stride, seq_lens, max_seq_len, nullptr, batch, k_tail, v_tail, softmax_scale,
      workspace, out, static_cast<hipStream_t>(stream)));
}

size_t kvarn_decode_noalloc_max_workspace_bytes(void) { return kvarn::kDecodeScratchBytes; }

kvarn_status kvarn_decode_attention_noalloc(const kvarn_params* params, const void* q,
                                            int32_t batch, int32_t num_q_heads,
                                            int32_t num_kv_heads, const void* k_pool,
                                            const void* v_pool, int64_t pool_num_pages,
                                            const int32_t* block_table,
                                            int32_t block_table_stride, const int32_t* seq_lens,
                                            int32_t max_seq_len, const void* k_tail,
                                            const void* v_tail, float softmax_scale, void* out,
                                            void* stream) {
  const kvarn_status st =
      check_decode(params, q, batch, num_q_heads, num_kv_heads, k_pool, v_pool, pool_num_pages,
                   block_table, block_table_stride, seq_lens, max_seq_len, k_tail, v_tail,
                   softmax_scale, out);
  if (st != KVARN_OK || batch == 0) return st;
  if (kvarn::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len) >
      kvarn::kDecodeScratchBytes)
    return KVARN_ERR_WORKSPACE;
  // the stream must belong to the current device, whose scratch copy the kernels use
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = 0, sdev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return KVARN_ERR_HIP;
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return KVARN_ERR_HIP;
    if (sdev != cur) return KVARN_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  if (kvarn::decode_scratch(&ws) != hipSuccess) return KVARN_ERR_HIP;
  return launch_status(kvarn::launch_decode(
      params->k_bits, params->v_bits, params->format, params->group, q, batch, num_q_heads, num_kv_heads, k_pool, v_pool,
      pool_num_pages, block_table, block_table_stride, seq_lens, max_seq_len, nullptr, batch,
      k_tail, v_tail, softmax_scale, ws, out, s));
}

kvarn_status kvarn_chunk_attention(const kvarn_params* params, const void* q, int32_t total_q,
                                   const int32_t* cu_q, int32_t batch, int32_t num_q_heads,
                                   int32_t num_kv_heads, const void* k_pool, const void* v_pool,
                                   int64_t pool_num_pages, const int32_t* block_table,
                                   int32_t block_table_stride, const int32_t* seq_lens,
                                   int32_t max_seq_len, const void* k_tail, const void* v_tail,
                                   float softmax_scale, void* workspace, size_t workspace_bytes,
                                   void* out, void* stream) {
  const kvarn_status st = kvarn_params_check(params);
  if (st != KVARN_OK) return st;
  if (total_q < 0 || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      pool_num_pages < 0 || block_table_stride < 0 || num_q_heads > 65535 || num_kv_heads > 65535)
    return KVARN_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return KVARN_ERR_INVALID_ARG;
  if (num_q_heads / num_kv_heads > kMaxGroup) return KVARN_ERR_UNSUPPORTED;
  if (total_q > 65535) return KVARN_ERR_UNSUPPORTED;      // one grid dimension per query row
  if (int64_t(total_q) * num_kv_heads > INT32_MAX) return KVARN_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale)) return KVARN_ERR_INVALID_ARG;
  if (total_q == 0) return KVARN_OK;
  if (batch == 0) return KVARN_ERR_INVALID_ARG;            // query rows without a sequence
  if (!q || !cu_q || !seq_lens || !out || !workspace) return KVARN_ERR_INVALID_ARG;
  if ((k_tail == nullptr) != (v_tail == nullptr)) return KVARN_ERR_INVALID_ARG;
  if (max_seq_len >= 128) {
    if (!k_pool || !v_pool || !block_table) return KVARN_ERR_INVALID_ARG;
    if (pool_num_pages * int64_t(num_kv_heads) > (int64_t(1) << 32)) return KVARN_ERR_UNSUPPORTED;
    if (block_table_stride < max_seq_len / 128) return KVARN_ERR_INVALID_ARG;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return KVARN_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVARN_ERR_INVALID_ARG;
  if (k_tail && (!aligned16(k_tail) || !aligned16(v_tail))) return KVARN_ERR_INVALID_ARG;
  if (workspace_bytes < kvarn::chunk_workspace_bytes(total_q, num_q_heads, num_kv_heads, max_seq_len))
    return KVARN_ERR_WORKSPACE;
  return launch_status(kvarn::launch_decode(
      params->k_bits, params->v_bits, params->format, params->group, q, total_q, num_q_heads, num_kv_heads, k_pool, v_pool, pool_num_pages, block_table,
      block_table_stride, seq_lens, max_seq_len, cu_q, batch, k_tail, v_tail, softmax_scale,
      workspace, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

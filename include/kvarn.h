/*
 * kvarn.h -- C ABI of the KVarN tile quantizer and paged decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (KVarN README, "How KVarN works", four stages): a KV cache is cut into
 * 128-token tiles (channels x tokens); each tile is rotated along channels by an
 * orthonormal Hadamard matrix, normalized by an iterative log-space Sinkhorn-style
 * alternation of column-std and row-std normalization, then quantized by asymmetric
 * round-to-nearest, keys 4-bit with scales per channel, values 2-bit with scales per token
 * (preset "kvarn_k4v2_g128", README "Quick start"; 128 = tile / page size). The presets
 * "kvarn_k2v2_g128" (2-bit keys; the pages report 2-bit results) and "kvarn_k4v4_g128"
 * (4-bit values; another key / value width choice of the same naming, README "How KVarN
 * works", the preset paragraph) are also implemented, and each of the three with group
 * size 64 ("_g64": keys in two 64-token groups per channel, values in two 64-channel groups
 * per token, each group with its own scale and zero; the finer setting of the group-size
 * knob the quick-start blog's configuration example describes).
 * The read path is decode attention that dequantizes the tiles on the fly: the query is
 * rotated by H for QK and the accumulated values are rotated back by H^T.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are DEVICE pointers owned by the caller; the library never
 *     frees or retains them. Host pointers are named *_host or are plain structs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). All GPU work
 *     is enqueued on it; calls return once the work is queued.
 *   - The library allocates no memory. It keeps no global state except the fixed decode
 *     scratch of kvarn_decode_attention_noalloc (one per GPU, below). It is re-entrant.
 *   - Arguments are validated on the host before anything is enqueued. On any error
 *     nothing is enqueued and outputs are untouched.
 *   - Device-resident indices (page ids, token offsets, sequence lengths) cannot be checked
 *     on the host; the kernels bound-check them and skip out-of-range entries instead of
 *     faulting (documented per call).
 *   - float16 is IEEE binary16, little-endian. Rounding to float16 is nearest-even.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points keep default visibility even when the library is built with hidden
 * visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define KVARN_API __attribute__((visibility("default")))
#else
#define KVARN_API
#endif

#define KVARN_ABI_VERSION 2
/* Page record formats (kvarn_params.format): */
#define KVARN_FORMAT_SEPARATE 1 /* normalizers and group scale / zero stored apart      */
#define KVARN_FORMAT_FOLDED 2   /* each group's normalizer folded into its scale / zero */
#define KVARN_FORMAT_VERSION KVARN_FORMAT_FOLDED   /* highest format this library reads  */

typedef enum {
    KVARN_OK = 0,
    KVARN_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misalignment, bad enum      */
    KVARN_ERR_UNSUPPORTED = 2, /* a valid request outside what this library implements */
    KVARN_ERR_WORKSPACE = 3,   /* workspace smaller than kvarn_decode_workspace_bytes */
    KVARN_ERR_HIP = 4          /* the HIP runtime refused a launch                    */
} kvarn_status;

typedef enum { KVARN_K = 0, KVARN_V = 1 } kvarn_kind;

/* Quantizer parameters. Only head_dim = tile_tokens = 128, group = 128 or 64, with
 * (k_bits, v_bits) = (4, 2), (2, 2) or (4, 4) are implemented (README "Quick start": other
 * page sizes are not yet supported). sinkhorn_iters is the number of (column step, row step) pairs of the
 * normalization (README "How KVarN works", stage 3); 0..64 accepted. format selects the page
 * record layout (KVARN_FORMAT_SEPARATE or KVARN_FORMAT_FOLDED, see kvarn_page_bytes);
 * kvarn_params_from_dtype sets KVARN_FORMAT_SEPARATE, anything else is INVALID_ARG. Every
 * call that reads or writes records must use the params the pool was written with. */
typedef struct {
    int32_t head_dim;
    int32_t tile_tokens;
    int32_t k_bits;
    int32_t v_bits;
    int32_t group;
    int32_t sinkhorn_iters;
    int32_t format;
} kvarn_params;

/* Library ABI version (KVARN_ABI_VERSION) and page-format version. */
KVARN_API int32_t kvarn_abi_version(void);
KVARN_API int32_t kvarn_format_version(void);

/* Human-readable name of a status code (static string, never NULL). */
KVARN_API const char* kvarn_status_str(kvarn_status status);

/* Parse a kv-cache dtype string of the form "kvarn_k<kb>v<vb>_g<group>" (README "Quick
 * start": kv_cache_dtype="kvarn_k4v2_g128") into params, with the given iteration count.
 * Returns INVALID_ARG for a malformed string or NULL pointer, UNSUPPORTED for a well-formed
 * preset other than k4v2, k2v2 and k4v4 with group 128 or 64. `out_host` is written only on
 * success. */
KVARN_API kvarn_status kvarn_params_from_dtype(const char* kv_cache_dtype, int32_t sinkhorn_iters,
                                     kvarn_params* out_host);

/* Check a params struct: OK, INVALID_ARG (NULL / out of range) or UNSUPPORTED. */
KVARN_API kvarn_status kvarn_params_check(const kvarn_params* params);

/* Bytes of one page record (one 128-token tile of one KV head) of the given kind: format
 * KVARN_FORMAT_SEPARATE 9216 for 4-bit keys or values, 5120 for 2-bit ones; format
 * KVARN_FORMAT_FOLDED 8960 and 4864; group 64 adds 512 to each (9728, 5632, 9472, 5376);
 * 0 if params are invalid or unsupported. Every pool passed with these params must use
 * this record size.
 *
 * Page format 1, KVARN_FORMAT_SEPARATE (little-endian):
 *   K record: bytes [0, 8192) are 4-bit codes, token-major: token t owns bytes
 *     [64t, 64t+64) as 16 32-bit words; word j holds channels 8j..8j+7 with nibble p
 *     (bits 4p..4p+3) holding channel 8j + {0,2,4,6,1,3,5,7}[p].
 *   V record: bytes [0, 4096) are 2-bit codes, channel-major: channel c owns the 8 words
 *     8c + 2g + d (g = 0..3, d = 0..1); crumb p (bits 2p..2p+1) of word (c, g, d) holds
 *     token 32 s + (j < 4 ? 4g + j : 12 + 4g + j) where i = p mod 8, s = 2d + i / 4,
 *     j = 2 (i mod 4) + p / 8.
 *   2-bit K record (k_bits = 2): bytes [0, 4096) are 2-bit codes, token-major: token t
 *     owns bytes [32t, 32t+32) as 8 32-bit words; word w = 2g + d holds channels
 *     16w .. 16w+15, crumb p (bits 2p..2p+1) holding channel 32g + 8(2d + p mod 8 / 4)
 *     + 2 (p mod 4) + p / 8.
 *   4-bit V record (v_bits = 4): bytes [0, 8192) are 4-bit codes, channel-major: channel c
 *     owns the 16 words 16c + 4g + m (g = 0..3, m = 0..3); nibble q (bits 4q..4q+3) of word
 *     (c, g, m) holds token 32 m + (j < 4 ? 4g + j : 12 + 4g + j), j = 2 (q mod 4) + q / 4
 *     (the 2-bit V record's token order, one nibble per code).
 *   All then hold four float16[128] vectors: r (per-channel normalizer), s (per-token
 *   normalizer), scale and zero (per channel for K, per token for V).
 *   A tile X (channels x tokens, rotated Xr = H X) is recovered as
 *     Xr[c][t] = r[c] * s[t] * (zero[g] + scale[g] * code[c][t]),  X = H Xr,
 *   with g = c for K and g = t for V, H the normalized natural-order Sylvester
 *   Hadamard matrix (symmetric, its own inverse).
 *
 * Page format 2, KVARN_FORMAT_FOLDED: the same code bytes, then three float16[128] vectors.
 * The group's own normalizer is folded into its scale and zero point, which are taken of
 * the tile divided by the other normalizer only (the asymmetric round-to-nearest of README
 * "How KVarN works" stage 4 is invariant to a positive factor per group):
 *   K record: s (per token), scale'[c], zero'[c] of Z = Xr / s per channel, so
 *     Xr[c][t] = s[t] * (zero'[c] + scale'[c] * code[c][t]);
 *   V record: r (per channel), scale'[t], zero'[t] of Z = Xr / r per token, so
 *     Xr[c][t] = r[c] * (zero'[t] + scale'[t] * code[c][t]).
 * 256 B fewer per record (3.6% of a k4v2 page pair).
 *
 * Group 64 (params.group = 64), either format: in place of one scale and one zero vector,
 * scale of half 0, scale of half 1, zero of half 0, zero of half 1 (each float16[128]), where
 * half h of a key channel c is tokens [64h, 64h + 64) and half h of a value token t is
 * channels [64h, 64h + 64): format 1 is codes, r, s, scale0, scale1, zero0, zero1; format 2
 * is codes, s (K) or r (V), scale'0, scale'1, zero'0, zero'1. Element (c, t) takes
 * g = (c, t / 64) for K and (t, c / 64) for V in the reconstruction above. */
KVARN_API size_t kvarn_page_bytes(const kvarn_params* params, kvarn_kind kind);

/* Quantize tiles into a page pool (README "How KVarN works", stages 1-4).
 *
 * For every tile i in [0, n_tiles) and KV head h in [0, num_kv_heads): the tile is
 * tokens [tile_src_token[i], tile_src_token[i] + 128) of head h of `src_dev`, element
 * (token, head, channel) at src_dev[token * src_token_stride + head * src_head_stride +
 * channel] (float16, strides in elements, channel stride 1). Its record is written to
 * pool_dev + (tile_dst_page[i] * num_kv_heads + h) * kvarn_page_bytes(params, kind).
 *
 * Arguments:
 *   src_dev: float16, 16-byte aligned; strides multiples of 8, non-negative.
 *   src_num_tokens: number of valid source tokens; tiles whose token range is not inside
 *     [0, src_num_tokens) are skipped (left unwritten).
 *   tile_src_token_dev: int64[n_tiles], tile_dst_page_dev: int32[n_tiles] (device).
 *   pool_dev: 16-byte aligned, pool_num_pages pages of num_kv_heads records; tiles whose
 *     page is outside [0, pool_num_pages) are skipped.
 *   n_tiles == 0 is a no-op returning OK.
 * Tiles must write distinct pages; overlapping destinations give an undefined record. */
KVARN_API kvarn_status kvarn_quantize_tiles(const kvarn_params* params, kvarn_kind kind,
                                  const void* src_dev, int64_t src_token_stride,
                                  int64_t src_head_stride, int64_t src_num_tokens,
                                  const int64_t* tile_src_token_dev,
                                  const int32_t* tile_dst_page_dev, int32_t n_tiles,
                                  int32_t num_kv_heads, void* pool_dev,
                                  int64_t pool_num_pages, void* stream);

/* Keys and values of the same tiles in one launch: exactly kvarn_quantize_tiles(KVARN_K) on
 * k_src_dev into k_pool_dev plus kvarn_quantize_tiles(KVARN_V) on v_src_dev into v_pool_dev
 * (same tile list), with every argument as described there. The two sources share strides
 * and token count; both pools have pool_num_pages pages of num_kv_heads records. A cache
 * write produces keys and values together; one launch keeps the GPU busy across both. */
KVARN_API kvarn_status kvarn_quantize_kv_tiles(const kvarn_params* params, const void* k_src_dev,
                                     const void* v_src_dev, int64_t src_token_stride,
                                     int64_t src_head_stride, int64_t src_num_tokens,
                                     const int64_t* tile_src_token_dev,
                                     const int32_t* tile_dst_page_dev, int32_t n_tiles,
                                     int32_t num_kv_heads, void* k_pool_dev, void* v_pool_dev,
                                     int64_t pool_num_pages, void* stream);

/* Append one decode token per sequence into the float16 staging tiles, and quantize every
 * staging tile that this append fills (the 128th token) into its page.
 *
 * For sequence b with L = seq_lens_dev[b] tokens BEFORE the append (0 <= L), the new
 * token k_new_dev[b][h][:] / v_new_dev[b][h][:] ([B, Hkv, 128] float16) is written to
 * row L mod 128 of k_tail_dev[b][h] / v_tail_dev[b][h] ([B, Hkv, 128, 128] float16,
 * [b][h][token][channel]). If L mod 128 == 127 the staging tiles of b are then quantized
 * (both kinds, all heads) into page block_table_dev[b * block_table_stride + L / 128] of
 * k_pool_dev / v_pool_dev. Pages outside [0, pool_num_pages) are skipped. The caller
 * increments seq_lens afterwards. Staging is plain float16 so the decode reads it exactly
 * (tiles are fixed-size, README "How KVarN works"; a partial tile is never quantized). */
KVARN_API kvarn_status kvarn_append_tokens(const kvarn_params* params, const void* k_new_dev,
                                 const void* v_new_dev, int32_t batch, int32_t num_kv_heads,
                                 const int32_t* seq_lens_dev, void* k_tail_dev,
                                 void* v_tail_dev, const int32_t* block_table_dev,
                                 int32_t block_table_stride, void* k_pool_dev,
                                 void* v_pool_dev, int64_t pool_num_pages, void* stream);

/* Write a chunk of new tokens per sequence into the cache: the prefill write path, with the
 * staging append fused in (README "Quick start": one page = one 128-token tile; "How KVarN
 * works": tiles are quantized whole, stages 1-4).
 *
 * Sequence b holds L = seq_lens_dev[b] tokens before the call (L >= 0; L < 0 skips b) and
 * receives n = cu_new_dev[b + 1] - cu_new_dev[b] tokens (clamped to [0, max_new_tokens]),
 * rows cu_new_dev[b] .. cu_new_dev[b] + n - 1 of k_new_dev / v_new_dev (float16
 * [total_new_tokens, num_kv_heads, 128], token-major, contiguous: the projection output), at
 * positions L .. L + n - 1. cu_new_dev: int32 [batch + 1], non-decreasing; a sequence whose
 * rows fall outside [0, total_new_tokens) is skipped. The host bound max_new_tokens >= every
 * n sizes the grid.
 *   - Every tile t completed by the chunk (L < 128 t + 128 <= L + n) is quantized, both kinds
 *     and all heads, into page block_table_dev[b * block_table_stride + t] of k_pool_dev /
 *     v_pool_dev. Rows of that tile below L are read from the staging tiles (the tile that
 *     was partial before the chunk), the others straight from k_new_dev / v_new_dev.
 *   - The chunk's tokens in the partial last tile (positions >= 128 floor((L+n)/128)) are
 *     written to rows (position mod 128) of k_tail_dev / v_tail_dev ([B, Hkv, 128, 128]
 *     float16); other staging rows are left as they are.
 * Tiles with t >= block_table_stride or a page outside [0, pool_num_pages) are skipped. The
 * caller advances seq_lens by n afterwards. With n = 1 this equals kvarn_append_tokens.
 * Two launches on `stream` (tiles, then staging); all pointers 16-byte aligned. */
KVARN_API kvarn_status kvarn_write_tokens(const kvarn_params* params, const void* k_new_dev,
                                const void* v_new_dev, int32_t total_new_tokens,
                                const int32_t* cu_new_dev, int32_t max_new_tokens,
                                int32_t batch, int32_t num_kv_heads,
                                const int32_t* seq_lens_dev, void* k_tail_dev, void* v_tail_dev,
                                const int32_t* block_table_dev, int32_t block_table_stride,
                                void* k_pool_dev, void* v_pool_dev, int64_t pool_num_pages,
                                void* stream);

/* Attention of several query positions per sequence over the quantized cache: the read path
 * of a prefill chunk (or of draft tokens to verify), causal, same arithmetic as
 * kvarn_decode_attention per query position (README intro: attention reads the quantized
 * cache; "How KVarN works" stage 4: scales re-applied on read).
 *
 * The cache of sequence b holds C = seq_lens_dev[b] tokens (clamped to [0, max_seq_len]), the
 * chunk already written into it (kvarn_write_tokens). Its query rows are
 * cu_q_dev[b] .. cu_q_dev[b + 1] - 1 of q_dev (float16 [total_q, num_q_heads, 128]): row
 * cu_q_dev[b] + i is position C - n + i, n = cu_q_dev[b + 1] - cu_q_dev[b], and attends to
 * positions 0 .. C - n + i (rows at positions below 0 get zeros). Positions in completed
 * tiles are read from the pages (a tile cut by the causal limit is read with a mask), those
 * of the partial last tile from the staging tiles (ignored when k_tail_dev / v_tail_dev are
 * NULL). out_dev: float16 [total_q, num_q_heads, 128]. cu_q_dev: int32 [batch + 1],
 * non-decreasing, cu_q_dev[0] = 0, cu_q_dev[batch] = total_q.
 * Limits and other arguments as kvarn_decode_attention with total_q in place of batch;
 * workspace_dev: >= kvarn_chunk_workspace_bytes(params, total_q, ...) bytes; total_q <= 65535
 * (UNSUPPORTED above). With one query row per sequence the read runs the decode kernels in
 * their split layout (the same result as kvarn_decode_attention up to float32 summation
 * order: a decode of several sequences balances its pages across waves instead); with more
 * rows than sequences a wave holds 16
 * query vectors (rows x heads of one sequence and KV head) and streams each page once for
 * all of them. */
KVARN_API kvarn_status kvarn_chunk_attention(const kvarn_params* params, const void* q_dev,
                                   int32_t total_q, const int32_t* cu_q_dev, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads,
                                   const void* k_pool_dev, const void* v_pool_dev,
                                   int64_t pool_num_pages, const int32_t* block_table_dev,
                                   int32_t block_table_stride, const int32_t* seq_lens_dev,
                                   int32_t max_seq_len, const void* k_tail_dev,
                                   const void* v_tail_dev, float softmax_scale,
                                   void* workspace_dev, size_t workspace_bytes, void* out_dev,
                                   void* stream);

/* Test and inspection only, off the hot path: page records back to float16 tiles (the read
 * side of README "How KVarN works" stage 4, then the inverse rotation; H is its own
 * inverse). For i < n_tiles and head h < num_kv_heads, the record (pages_dev[i], h) of
 * pool_dev (pool_num_pages pages of num_kv_heads records of kind `kind`) becomes
 *   dst_dev[i][h][t][c] = f16_rne( (H Xr)[c][t] ),  Xr[c][t] = r[c] s[t] (zero[g] + scale[g] code[c][t])
 * (g = c for keys, t for values; evaluated in float32). dst_dev: float16
 * [n_tiles, num_kv_heads, 128, 128], 16-byte aligned; pool_dev 16-byte aligned. Pages
 * outside [0, pool_num_pages) leave their dst tile untouched. n_tiles == 0 is a no-op. */
KVARN_API kvarn_status kvarn_dequantize_tiles(const kvarn_params* params, kvarn_kind kind,
                                    const void* pool_dev, int64_t pool_num_pages,
                                    const int32_t* pages_dev, int32_t n_tiles,
                                    int32_t num_kv_heads, void* dst_dev, void* stream);

/* Workspace bytes kvarn_decode_attention needs for this shape (0 if invalid). */
KVARN_API size_t kvarn_decode_workspace_bytes(const kvarn_params* params, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_seq_len);

/* Workspace bytes kvarn_chunk_attention needs for total_q query rows (0 if invalid). */
KVARN_API size_t kvarn_chunk_workspace_bytes(const kvarn_params* params, int32_t total_q,
                                   int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_seq_len);

/* Number of key splits per (sequence, KV head) of the split layout for this shape (0 if
 * invalid); informative. The split layout serves a decode of one sequence and chunk reads
 * with one query row per sequence. A decode of 2 .. 1024 sequences instead gives every wave
 * of one round (2,048 waves) an equal share of all (sequence, KV head, page) entries. */
KVARN_API int32_t kvarn_decode_num_splits(const kvarn_params* params, int32_t batch,
                                int32_t num_kv_heads, int32_t max_seq_len);

/* Paged decode attention over quantized pages plus a float16 tail (README intro: a native
 * attention backend reading the quantized cache; "How KVarN works" stage 4: scales are
 * re-applied on read).
 *
 * For sequence b, query head hq, KV head g = hq / (num_q_heads / num_kv_heads):
 *   L = min(seq_lens_dev[b], max_seq_len); pages p < L / 128 are
 *   block_table_dev[b * block_table_stride + p] of k_pool_dev / v_pool_dev; the last
 *   L mod 128 tokens are rows 0.. of k_tail_dev[b][g] / v_tail_dev[b][g].
 *   out[b][hq] = sum_t softmax_t(softmax_scale * q[b][hq] . k_t) v_t  (float16, RNE),
 *   k_t, v_t the dequantized (or staged) keys and values.
 * Arguments:
 *   q_dev, out_dev: [batch, num_q_heads, 128] float16, contiguous, 16-byte aligned.
 *   num_q_heads % num_kv_heads == 0 and num_q_heads / num_kv_heads <= 8.
 *   batch <= 65535 and batch * num_kv_heads <= INT32_MAX (grid limits; UNSUPPORTED above).
 *   k_tail_dev / v_tail_dev may be NULL: then tail tokens are ignored. Staging rows from
 *   L mod 128 on are never read (they may hold anything, NaN included).
 *   Pages outside [0, pool_num_pages) are skipped. A sequence with L = 0, or with every
 *   page skipped and no tail, gets out = 0.
 *   workspace_dev: >= kvarn_decode_workspace_bytes(...) bytes, 16-byte aligned; it holds
 *   per-split partial softmax state and must not be shared by concurrent calls. */
KVARN_API kvarn_status kvarn_decode_attention(const kvarn_params* params, const void* q_dev,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    const void* k_pool_dev, const void* v_pool_dev,
                                    int64_t pool_num_pages, const int32_t* block_table_dev,
                                    int32_t block_table_stride, const int32_t* seq_lens_dev,
                                    int32_t max_seq_len, const void* k_tail_dev,
                                    const void* v_tail_dev, float softmax_scale,
                                    void* workspace_dev, size_t workspace_bytes,
                                    void* out_dev, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): kvarn_decode_attention without a workspace argument.
 * Every argument, the result and every error are those of kvarn_decode_attention; the
 * split partials live in a fixed device scratch buffer of
 * kvarn_decode_noalloc_max_workspace_bytes() bytes (32 MiB) that the library holds on each
 * GPU it runs on until the process ends. A shape whose kvarn_decode_workspace_bytes exceeds
 * it returns KVARN_ERR_WORKSPACE with nothing enqueued. The call allocates no memory; its
 * first call on a device looks up that device's scratch address (KVARN_ERR_HIP on failure).
 * `stream` must belong to the current device (KVARN_ERR_INVALID_ARG otherwise). The scratch
 * needs no clearing (every partial the merge reads is written by the same call). All calls
 * on one GPU share its scratch: calls that overlap in time on one GPU (concurrent streams,
 * or host threads enqueueing on different streams) race and give undefined output; calls
 * ordered on one stream are safe. */
KVARN_API size_t kvarn_decode_noalloc_max_workspace_bytes(void);
KVARN_API kvarn_status kvarn_decode_attention_noalloc(const kvarn_params* params,
                                            const void* q_dev, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            const void* k_pool_dev, const void* v_pool_dev,
                                            int64_t pool_num_pages,
                                            const int32_t* block_table_dev,
                                            int32_t block_table_stride,
                                            const int32_t* seq_lens_dev, int32_t max_seq_len,
                                            const void* k_tail_dev, const void* v_tail_dev,
                                            float softmax_scale, void* out_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */

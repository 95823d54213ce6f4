// Host-side functions one source file of the library calls in another (not
// exported: the C ABI is include/pa.h).
#pragma once

#include "pa_device.h"

namespace pa {

// decode.hip: start-up units per (sequence, KV head group) segment of the
// decode work split (units are 16-token steps), by cache dtype; the bound
// DECODE_SEG_OV_MAX is what the host's unit-count checks use (prefill.hip
// checks its decode rows' units with it).
__host__ __device__ constexpr int decode_seg_ov(int cache_dtype) {
  return cache_dtype == PA_F32 || cache_dtype == PA_BF16 ? 2 : 6;
}
constexpr int DECODE_SEG_OV_MAX = 6;

// decode.hip: chunked prefill over an fp32 cache, each query row run as a
// decode row of its chunk's sequence on the vector decode kernel.
size_t prefill_f32_workspace_bytes(int total_q, int n_kv, int G, int head_dim,
                                   int max_context_len);
pa_status prefill_f32_rows(float* out, const float* q, const int32_t* cu_seqlens_q, int num_seqs,
                           int total_q, const void* k_cache, const void* v_cache, int num_blocks,
                           int block_size, int n_kv, int head_dim, int G,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int max_context_len, int causal,
                           float scale, void* workspace, size_t workspace_bytes, hipStream_t st);

// decode.hip: the query-length-1 rows of a chunked-prefill batch on the
// matrix-core decode path.  row_ctx[s] is sequence s's context when its chunk
// is one query long and 0 otherwise; row_map[s] is that query's row of q and
// out, or -1 (the merge writes no output for the sequence).  Needs
// block_size >= 16 and a bf16 query; the workspace holds the split partials.
size_t prefill_decode_rows_workspace_bytes(int num_seqs, int n_kv, int G, int head_dim);
pa_status prefill_decode_rows(void* out, const void* q, const void* k_cache, const void* v_cache,
                              int cache_dtype, int num_blocks, int block_size, int n_kv,
                              int head_dim, int G, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* row_ctx,
                              const int32_t* row_map, int num_seqs, int max_context_len,
                              float scale, float k_scale, float v_scale,
                              const float* k_channel_scales, const float* v_token_scales,
                              void* workspace, size_t workspace_bytes, hipStream_t st);

}  // namespace pa

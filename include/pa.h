/*
 * pa.h -- C ABI of the paged-KV attention library (libpa.so, gfx950 / MI355X).
 *
 * The operations follow the paged KV cache of the pages this library is built
 * from:
 *   - "3.3 Batching and memory management" (llm-learning-path tutorial),
 *     section "PagedAttention: the block table": the KV pool is cut into
 *     physical blocks of block_size tokens; entry j of a sequence's block
 *     table names the block holding its tokens [j*block_size, (j+1)*block_size);
 *     token p lives in block table[p / block_size] at offset p % block_size.
 *     Section "Chunked prefill": a chunk's queries attend to a cache that
 *     already holds the earlier chunks.
 *   - "KV Cache: the memory bottleneck of LLM inference" (excerpt on the
 *     "PagedAttention" tag page), section 1.1: at step t the new k_t, v_t are
 *     appended to the cache and the output is softmax(q_t K_{1:t}^T/sqrt(d)) V_{1:t}.
 *   - "From PagedAttention to Chunked Prefill" (ybb.press), section 2.2: the
 *     kernel walks the blocks with the online (iterative) softmax recurrence;
 *     section 3.2: one batch mixes query_len = 1 decode rows and
 *     query_len = chunk prefill rows, located by cumulative offsets.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer owned by the caller.
 *   The library allocates no device memory, keeps no per-call state and never
 *   synchronises: each call enqueues its kernels on `stream` (a hipStream_t;
 *   NULL = the null stream) and returns.  Calls on different streams may run
 *   concurrently when their output buffers do not overlap.
 * Cache layout.  k_cache and v_cache are per-layer pools, row-major
 *   [num_blocks][block_size][n_kv_heads][head_dim] of `cache_dtype` elements.
 * Block tables.  int32 [num_seqs][max_blocks_per_seq], row-major; only the
 *   first ceil(context_len / block_size) entries of a row are read; padding
 *   entries should be -1.
 * Context lengths.  int32 [num_seqs]; context_lens[s] counts every token of
 *   sequence s INCLUDING the ones appended in the current step (append first,
 *   then attend).
 * Heads.  n_q_heads = n_kv_heads * group_size; query head h reads KV head
 *   h / group_size (grouped-query attention; group_size 1 is multi-head).
 * Errors.  Host-checkable errors return a status before anything is enqueued;
 *   a failed launch returns PA_ERR_HIP.  Device-resident preconditions are not
 *   checked on the device: block ids must lie in [0, num_blocks) for the
 *   positions that are read, context_lens[s] <= max_blocks_per_seq*block_size,
 *   context_lens[s] <= max_context_len, append slots must be distinct.  As a
 *   guard against memory faults only, an append slot outside the pool is not
 *   written, and attention reads through a block id outside the pool go to
 *   block 0 instead: the output rows of such a sequence are unspecified, but
 *   no access leaves the pools.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,        /* inconsistent or negative sizes */
  PA_ERR_DTYPE = 3,        /* unsupported dtype or dtype pair */
  PA_ERR_UNSUPPORTED = 4,  /* head_dim / block_size / group_size outside the supported set */
  PA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than the query function says */
  PA_ERR_HIP = 6           /* a HIP launch or runtime call failed */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,              /* IEEE binary32 */
  PA_BF16 = 1,             /* bfloat16 */
  PA_FP8_E4M3 = 2,         /* OCP FP8 E4M3 (e4m3fn: bias 7, max 448, no inf, NaN = 0x7F/0xFF) */
  PA_INT8 = 3,             /* symmetric int8 codes in [-127, 127] (cache only) */
  PA_INT4 = 4              /* symmetric 4-bit codes in [-7, 7], two per byte (cache only;
                              the *_int4 entry points and pa_copy_blocks) */
} pa_dtype;

/* Human-readable name of a status code.  Never NULL. */
const char* pa_status_string(int status);

/* ABI version of this header (bumped on any signature change). */
int pa_abi_version(void);

/*
 * pa_slot_mapping -- the block-table address map for a ragged set of tokens.
 *   Source: "3.3 Batching and memory management", section "PagedAttention:
 *   the block table" (physical block = table[p / block_size], offset =
 *   p mod block_size).
 *
 *   Token i of segment s (cu_tokens[s] <= i < cu_tokens[s+1]) sits at logical
 *   position p = start_pos[s] + (i - cu_tokens[s]) of sequence s and gets
 *     slot_mapping[i] = table[s][p / block_size] * block_size + p % block_size,
 *   or -1 when that table entry is negative.  Decode rows use
 *   start_pos = context_len - 1 and one token; a prefill chunk of L tokens uses
 *   start_pos = context_len - L.
 *
 *   slot_mapping  int64 [num_tokens]      (out)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   cu_tokens     int32 [num_seqs + 1]    cumulative token counts, cu_tokens[num_seqs] == num_tokens
 *   start_pos     int32 [num_seqs]
 *   block_size    >= 1 (any value)
 *   Positions past the table row (p / block_size >= max_blocks_per_seq) give -1.
 */
pa_status pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t block_size,
                          const int32_t* cu_tokens, const int32_t* start_pos,
                          int32_t num_seqs, int32_t num_tokens, void* stream);

/*
 * pa_kv_append -- scatter new K/V rows into their cache slots.
 *   Source: "KV Cache: the memory bottleneck of LLM inference", section 1.1
 *   (append k_t, v_t to the cache); slot addressing as in pa_slot_mapping.
 *
 *   For every i with 0 <= slot_mapping[i] < num_blocks*block_size:
 *     k_cache[slot / block_size][slot % block_size][h][:] = enc(k_new[i][h][:])  (all h)
 *   and the same for V.  Negative slots are skipped; no other byte of the
 *   pools is written.  enc is a bit copy when src_dtype == cache_dtype
 *   (F32 or BF16); for an FP8_E4M3 cache (src F32 or BF16) it is
 *     e4m3_satfinite_rne( float(x) * (1.0f / scale) )
 *   with the inverse computed once in binary32 on the host, the magnitude
 *   clamped to 448 (infinities too), ties rounded to even, NaN -> 0x7F; for
 *   an INT8 cache (src F32 or BF16; the 8-bit step of "From PagedAttention to
 *   Chunked Prefill", section 5.4) it is
 *     clamp(rint_ties_even( float(x) * (1.0f / scale) ), -127, 127)
 *   with NaN -> 0.
 *   k_scale / v_scale are the per-tensor scales (read only for FP8 and INT8
 *   caches).
 *
 *   k_new, v_new  [num_tokens][n_kv_heads][head_dim] of src_dtype (contiguous)
 *   slot_mapping  int64 [num_tokens], distinct non-negative entries
 *   head_dim      a multiple of 8; num_tokens * n_kv_heads * head_dim / 8 < 2^31
 *                 (else PA_ERR_SHAPE)
 */
pa_status pa_kv_append(void* k_cache, void* v_cache, int cache_dtype,
                       int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                       int32_t head_dim, const void* k_new, const void* v_new,
                       int src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                       float k_scale, float v_scale, void* stream);

/*
 * pa_kv_append_paged -- pa_slot_mapping and pa_kv_append in one launch.
 *   Source: the block-table address map of "3.3 Batching and memory
 *   management", section "PagedAttention: the block table", and the append of
 *   "KV Cache: the memory bottleneck of LLM inference", section 1.1.
 *
 *   Token i of segment s (cu_tokens[s] <= i < cu_tokens[s+1]) gets the slot
 *   pa_slot_mapping gives it (from block_tables, start_pos, block_size) and is
 *   appended exactly as pa_kv_append appends it with that slot: same encoders,
 *   same skipping of negative and out-of-pool slots, bit-identical pools.
 *   slot_mapping (int64 [num_tokens], may be NULL) receives the slots as
 *   pa_slot_mapping writes them.
 *
 *   max_tokens_per_seq  host-side bound on the segment lengths; it sizes the
 *                       grid only (longer segments are still appended whole)
 *   cu_tokens           int32 [num_seqs + 1], non-decreasing, last entry
 *                       num_tokens; token indices outside [0, num_tokens) are
 *                       never read or written
 *   other arguments     as in pa_slot_mapping and pa_kv_append
 */
pa_status pa_kv_append_paged(void* k_cache, void* v_cache, int cache_dtype,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t head_dim, const void* k_new, const void* v_new,
                             int src_dtype, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* cu_tokens,
                             const int32_t* start_pos, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_tokens_per_seq, int64_t* slot_mapping,
                             float k_scale, float v_scale, void* stream);

/*
 * pa_decode_workspace_bytes -- scratch needed by pa_decode for these sizes.
 *   split_tokens: 0 = the library's choice; otherwise the minimum number of
 *   context tokens one split (one workgroup) handles, rounded up to 16.
 *   The same split_tokens must be passed to pa_decode.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t split_tokens);

/*
 * pa_decode -- single-token paged attention for a ragged batch.
 *   Source: attention at step t over K_{1:t}, V_{1:t} ("KV Cache: the memory
 *   bottleneck", section 1.1) gathered through the block table ("3.3 Batching
 *   and memory management", "PagedAttention: the block table"), computed
 *   block by block with the online softmax recurrence ("From PagedAttention to
 *   Chunked Prefill", section 2.2; rescale factor e^{m_old - m_new} applied
 *   to the unnormalised accumulator, division by the running sum at the end).
 *   Long contexts are cut into splits handled by separate workgroups; their
 *   partial (m, l, O) are combined with the log-sum-exp merge
 *   M = max m_k, O = sum_k e^{m_k - M} O_k / sum_k e^{m_k - M} l_k.
 *
 *   out[s][h][:] = sum_j softmax_j(scale * q[s][h] . K_s[j][h/g]) V_s[j][h/g][:],
 *   j < context_lens[s]; a sequence with context 0 gets zeros.  For FP8 and
 *   INT8 caches the stored codes are multiplied by k_scale / v_scale.
 *
 *   out           [num_seqs][n_q_heads][head_dim], dtype = q_dtype (bf16 output is
 *                 rounded to nearest even)
 *   q             [num_seqs][n_q_heads][head_dim] of q_dtype
 *   dtype pairs   (q, cache) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 *                 (BF16, INT8)}
 *   head_dim      64 or 128;  block_size a power of two in [1, 256];
 *   group_size    1, 2, 4 or 8
 *   max_context_len  host-side upper bound of context_lens (sizes the plan)
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...)
 *                 bytes, 256-byte aligned; contents need no initialisation and
 *                 are clobbered.
 *   Results are deterministic run to run (no atomics) and do not depend on
 *   which physical blocks hold the tokens.
 */
pa_status pa_decode(void* out, const void* q, int q_dtype,
                    const void* k_cache, const void* v_cache, int cache_dtype,
                    int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                    int32_t head_dim, int32_t group_size,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                    float scale, float k_scale, float v_scale, int32_t split_tokens,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_workspace_bytes -- scratch needed by pa_prefill_chunk (0 for an
 * empty batch or unsupported head counts), for either dtype pair and any block
 * size (it includes the split partials of the rows of length 1).  It grows
 * with num_seqs and total_q, not with num_seqs times max_q_len: a batch of
 * many decode rows beside a few long chunks needs little.  The call must pass the same
 * num_seqs, total_q and max_q_len.
 */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                  int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                  int32_t max_context_len);

/*
 * pa_prefill_chunk -- attention of ragged query chunks over the paged cache.
 *   Source: "3.3 Batching and memory management", section "Chunked prefill"
 *   (a chunk's queries attend to a cache that already holds the earlier
 *   chunks); "From PagedAttention to Chunked Prefill", section 3.2 (one batch
 *   of rows with different query lengths, located by cumulative offsets) and
 *   section 2.2 (online softmax over key blocks); addressing as in pa_decode.
 *
 *   Chunk s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) (L_s rows);
 *   its cache holds T_s = context_lens[s] tokens, the chunk's own K/V included
 *   (appended first).  Query row i of the chunk sits at position T_s - L_s + i
 *   and attends to keys j <= T_s - L_s + i when causal != 0, to all j < T_s
 *   otherwise:
 *     out[row][h][:] = sum_j softmax_j(scale * q[row][h] . K_s[j][h/g]) V_s[j][h/g][:].
 *   A decode row is the special case L_s = 1, so one call serves a mixed
 *   step: prefill chunks and decode rows side by side, in any order -- the
 *   engine's view in "From PagedAttention to Chunked Prefill", section 3.2.
 *   Inside the call a planning launch lists the chunks' work, the tile launch
 *   spreads it over the device in equal shares of 32-key tiles, and a merge
 *   launch combines split tiles.  With blocks of 16 tokens or more the rows
 *   of length 1 are left out of the tiles and run on pa_decode's split and
 *   merge launches instead (whole token rows streamed through the matrix
 *   cores; the planner lists them on the device, so the host reads nothing).
 *
 *   (q, cache) dtype pairs: (BF16, BF16), (BF16, FP8_E4M3), (BF16, INT8) on
 *   the matrix cores, and (F32, F32), where each query row runs as a decode
 *   row of its chunk's sequence (context T_s - L_s + i + 1 when causal, T_s
 *   otherwise) on the fp32 vector decode kernel.
 *
 *   out, q        [total_q][n_q_heads][head_dim] of q_dtype (BF16 or F32)
 *   cu_seqlens_q  int32 [num_seqs + 1], non-decreasing, cu_seqlens_q[num_seqs] == total_q
 *   max_q_len     host-side upper bound of the L_s.  A cu_seqlens_q that
 *                 needs more query tiles than total_q and max_q_len allow
 *                 (the device-side planner checks) is not computed: out is
 *                 left unwritten and nothing outside the arguments is touched.
 *   cache_dtype   BF16, FP8_E4M3 or INT8 (codes times k_scale / v_scale) with
 *                 BF16 queries; F32 with F32 queries
 *   head_dim      64 or 128; block_size a power of two in [1, 256];
 *                 block_size * n_kv_heads * head_dim * 2 below 2^31 (a block's
 *                 rows are addressed with 32-bit offsets), else PA_ERR_SHAPE
 *   group_size    1, 2, 4 or 8
 *   scale         positive and finite, else PA_ERR_SHAPE
 *   max_context_len  upper bound of the T_s; with block_size >= 16,
 *                 num_seqs * n_kv_heads * ceil(max_context_len / 16) below 2^31
 *                 (the decode path's units), else PA_ERR_SHAPE
 *   workspace     at least pa_prefill_workspace_bytes(...) bytes (may be NULL if 0)
 */
pa_status pa_prefill_chunk(void* out, const void* q, int q_dtype,
                           const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t total_q,
                           int32_t max_q_len, const void* k_cache, const void* v_cache,
                           int cache_dtype, int32_t num_blocks, int32_t block_size,
                           int32_t n_kv_heads, int32_t head_dim, int32_t group_size,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len,
                           int32_t causal, float scale, float k_scale, float v_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partials / pa_decode_merge -- the two phases of pa_decode, for
 * callers that schedule them apart: timing the split kernel alone, or running
 * the merge after partials from several devices (each holding a slice of a
 * long context) have been gathered into one workspace.
 *
 * pa_decode_partials takes pa_decode's arguments minus `out` and `v_scale` and
 * leaves, per (sequence, query head, split), the split's running maximum m
 * (base-2 logarithm units of the scaled scores), its sum l and its
 * unnormalised accumulator O in the workspace.  The workspace layout is
 * private to this library version; only pa_decode_merge reads it.
 *
 * pa_decode_merge combines them (M = max m_k, out = out_scale * sum_k 2^{m_k-M} O_k /
 * sum_k 2^{m_k-M} l_k; zeros for context 0) and writes `out` in out_dtype (F32
 * or BF16).  out_scale is v_scale for FP8 and INT8 caches and 1 otherwise.  It must be
 * called with the num_seqs, head counts, head_dim, max_context_len,
 * split_tokens and context_lens of the partials call it follows.
 */
pa_status pa_decode_partials(const void* q, int q_dtype,
                             const void* k_cache, const void* v_cache, int cache_dtype,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t head_dim, int32_t group_size,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, float scale, float k_scale,
                             int32_t split_tokens, void* workspace, size_t workspace_bytes,
                             void* stream);

pa_status pa_decode_merge(void* out, int out_dtype, const int32_t* context_lens,
                          int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, int32_t max_context_len, int32_t split_tokens,
                          float out_scale, const void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * pa_decode_append / pa_decode_append_partials -- the decode step's append and
 *   attention in one call: every sequence's newest token (position
 *   context_lens[s] - 1, the token this step added) is written to its cache slot
 *   and attended to.
 *   Source: "KV Cache: the memory bottleneck of LLM inference", section 1.1
 *   (step t appends k_t, v_t, then attends over K_{1:t}, V_{1:t}); slot
 *   addressing of "3.3 Batching and memory management", section
 *   "PagedAttention: the block table"; attention as in pa_decode.
 *
 *   Equivalent to pa_kv_append_paged (one token per sequence, start_pos =
 *   context_lens[s] - 1, cu_tokens = 0, 1, ..., num_seqs) followed by pa_decode
 *   (or pa_decode_partials): the same pools, slots and outputs, bit for bit.
 *   Where the split kernel stages whole rows (bf16, fp8 and int8 caches with
 *   blocks of 16 tokens or more) the append happens inside the attention
 *   launch: the workgroup that reads a sequence's newest token takes it from
 *   k_new / v_new and writes it to its slot.  Elsewhere the rows are written
 *   by a launch of their own first.
 *
 *   k_new, v_new  [num_seqs][n_kv_heads][head_dim] of src_dtype, 16-byte aligned
 *   src_dtype     = cache_dtype for F32 and BF16 caches; F32 or BF16 for
 *                 FP8_E4M3 and INT8 caches (encoded with k_scale / v_scale as
 *                 pa_kv_append does); INT4 caches: PA_ERR_DTYPE
 *   slot_mapping  int64 [num_seqs] (may be NULL): the slot each token was
 *                 written to, -1 for a negative table entry, a position past the
 *                 table row or a sequence with context 0 (nothing appended)
 *   k_cache, v_cache are written (the appended slots only); other arguments
 *   as in pa_decode / pa_decode_partials.  pa_decode_append_partials also takes
 *   v_scale (for the encode); pa_decode_merge applies it as out_scale.
 */
pa_status pa_decode_append(void* out, const void* q, int q_dtype,
                           void* k_cache, void* v_cache, int cache_dtype,
                           int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                           int32_t head_dim, int32_t group_size,
                           const void* k_new, const void* v_new, int src_dtype,
                           int64_t* slot_mapping,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, float scale, float k_scale, float v_scale,
                           int32_t split_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

pa_status pa_decode_append_partials(const void* q, int q_dtype,
                                    void* k_cache, void* v_cache, int cache_dtype,
                                    int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t group_size,
                                    const void* k_new, const void* v_new, int src_dtype,
                                    int64_t* slot_mapping,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t max_context_len, float scale, float k_scale,
                                    float v_scale, int32_t split_tokens, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * pa_decode_no_alloc -- pa_decode for callers that cannot allocate device
 *   memory: code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc.  Same arguments, results and checks as pa_decode, minus
 *   the workspace: the split partials go to a scratch array of
 *   PA_NO_ALLOC_SCRATCH_BYTES that the library holds on each device it runs
 *   on (a device variable, resident until the process ends; its address is
 *   looked up once per device on the first call there).  The call allocates
 *   nothing and needs no initialised scratch.
 *   A call whose partials (pa_decode_workspace_bytes(...) for its sizes) do
 *   not fit returns PA_ERR_WORKSPACE before anything is enqueued; use
 *   pa_decode with a workspace then.  All calls on one device share its
 *   scratch: calls that may overlap on one device (different streams, or
 *   different host threads without ordering) race and must be serialised by
 *   the caller.
 */
#define PA_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_no_alloc(void* out, const void* q, int q_dtype,
                             const void* k_cache, const void* v_cache, int cache_dtype,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t head_dim, int32_t group_size,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, float scale, float k_scale,
                             float v_scale, int32_t split_tokens, void* stream);

/*
 * pa_copy_blocks -- whole-block copies between paged pools: copy-on-write
 *   within one pool, and swap-out / swap-in between a device pool and a pool
 *   in pinned host memory.
 *   Source: "3.3 Batching and memory management", section "Sharing and
 *   copy-on-write" (a block that other sequences still reference is copied
 *   to a fresh block before one of them writes into it) and section
 *   "Scheduling policy and preemption" (a preempted sequence's blocks are
 *   copied out to host memory and copied back when it resumes).
 *
 *   For every pair i with 0 <= src < src_num_blocks and 0 <= dst < dst_num_blocks
 *   (block_pairs[2i] = src, block_pairs[2i+1] = dst):
 *     dst_k[dst][:][:][:] = src_k[src][:][:][:],  dst_v[dst] = src_v[src]
 *   byte for byte; other pairs are skipped and no other block is written.
 *
 *   dst_k, dst_v  [dst_num_blocks][block_size][n_kv_heads][head_dim] of cache_dtype
 *   src_k, src_v  [src_num_blocks][block_size][n_kv_heads][head_dim] of cache_dtype;
 *                 either pair of pools may be device memory or pinned host memory
 *                 (hipHostMalloc), which the kernel accesses directly; the src and
 *                 dst pools may be the same pools.
 *   block_pairs   int64 [num_pairs][2] in device memory.  Destinations distinct,
 *                 and no block is both a source and a destination in one call
 *                 (else which copy lands is unspecified).
 *   Pool bases 16-byte aligned (8 when a block's byte size is not a multiple
 *   of 16; a block's byte size must be a multiple of 8), else PA_ERR_SHAPE /
 *   PA_ERR_UNSUPPORTED.
 */
pa_status pa_copy_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks,
                         const void* src_k, const void* src_v, int32_t src_num_blocks,
                         int cache_dtype, int32_t block_size, int32_t n_kv_heads,
                         int32_t head_dim, const int64_t* block_pairs, int32_t num_pairs,
                         void* stream);

/*
 * INT4 KV cache -- "From PagedAttention to Chunked Prefill", section 5.4
 * (4-bit caches with KIVI's grouping: keys quantised along the channel axis,
 * values along the token axis).
 *
 *   Codes: symmetric integers in [-7, 7], two per byte, element 2i in the low
 *   nibble of byte i, each nibble sign-magnitude (8 * [c < 0] + |c|; the
 *   nibble 8 reads as 0).  The pools are [num_blocks][block_size][n_kv_heads]
 *   [head_dim / 2] bytes (cache_dtype PA_INT4 in pa_copy_blocks).
 *   Keys: k = code * k_channel_scales[h][d] (float32 [n_kv_heads][head_dim],
 *   device memory, from the caller's calibration).
 *   Values: v = code * v_scales[slot / block_size][h][slot % block_size]
 *   (float32 [num_blocks][n_kv_heads][block_size], device memory, written by
 *   the append beside the codes: one scale per token and head, the scales of
 *   one head's tokens of a block adjacent).  Moving a block (copy-on-write,
 *   swap) moves its codes and its v_scales block.
 *
 * pa_kv_append_int4 -- for every i with 0 <= slot_mapping[i] <
 * num_blocks * block_size and every head h:
 *   key codes   clamp(rint_ties_even(float(k) * (1.0f / k_channel_scales[h][d])), -7, 7)
 *   value scale sigma = a / 7.0f, a = max_d |v[i][h][d]| (NaN elements ignored)
 *   value codes clamp(rint_ties_even(float(v) * (1.0f / sigma)), -7, 7)
 * with NaN products encoding 0 (an all-zero row gets sigma 0 and codes 0), each
 * division one binary32 division.  k_new, v_new [num_tokens][n_kv_heads]
 * [head_dim] of src_dtype F32 or BF16; head_dim 64 or 128.  Other bytes and
 * scales are not written.
 */
pa_status pa_kv_append_int4(void* k_cache, void* v_cache, float* v_scales, int32_t num_blocks,
                            int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                            const void* k_new, const void* v_new, int src_dtype,
                            const int64_t* slot_mapping, int32_t num_tokens,
                            const float* k_channel_scales, void* stream);

/*
 * pa_kv_append_int4_paged -- pa_slot_mapping and pa_kv_append_int4 in one
 * launch, as pa_kv_append_paged is for pa_kv_append: bit-identical codes and
 * value scales; slot_mapping (may be NULL) receives the slots.
 */
pa_status pa_kv_append_int4_paged(void* k_cache, void* v_cache, float* v_scales,
                                  int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                  int32_t head_dim, const void* k_new, const void* v_new,
                                  int src_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* cu_tokens,
                                  const int32_t* start_pos, int32_t num_seqs,
                                  int32_t num_tokens, int32_t max_tokens_per_seq,
                                  int64_t* slot_mapping, const float* k_channel_scales,
                                  void* stream);

/*
 * pa_decode_int4 / pa_decode_int4_partials -- pa_decode and pa_decode_partials
 * over an INT4 cache (q_dtype BF16; no per-tensor scales).  The output is the
 * attention over the dequantised keys and values above.  In the kernel the
 * key scales multiply the query (rounded to bf16) and each value scale
 * multiplies its token's softmax weight (rounded to bf16); the sum l is
 * taken over the unscaled weights in fp32.  The workspace is
 * pa_decode_workspace_bytes(...); the partials are merged by pa_decode_merge
 * with out_scale 1.  pa_decode and pa_decode_partials return PA_ERR_DTYPE for
 * cache_dtype PA_INT4.
 */
pa_status pa_decode_int4(void* out, const void* q, int q_dtype, const void* k_cache,
                         const void* v_cache, const float* k_channel_scales,
                         const float* v_scales, int32_t num_blocks, int32_t block_size,
                         int32_t n_kv_heads, int32_t head_dim, int32_t group_size,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                         float scale, int32_t split_tokens, void* workspace,
                         size_t workspace_bytes, void* stream);

pa_status pa_decode_int4_partials(const void* q, int q_dtype, const void* k_cache,
                                  const void* v_cache, const float* k_channel_scales,
                                  const float* v_scales, int32_t num_blocks, int32_t block_size,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t group_size,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, float scale, int32_t split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_chunk_int4 -- pa_prefill_chunk over an INT4 cache (q_dtype BF16;
 * the key and value scales as for pa_decode_int4, no per-tensor scales).  The
 * output is the chunk attention over the dequantised keys and values.  The
 * workspace is pa_prefill_workspace_bytes(...); pa_prefill_chunk returns
 * PA_ERR_DTYPE for cache_dtype PA_INT4.
 */
pa_status pa_prefill_chunk_int4(void* out, const void* q, int q_dtype,
                                const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t total_q,
                                int32_t max_q_len, const void* k_cache, const void* v_cache,
                                const float* k_channel_scales, const float* v_scales,
                                int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                int32_t head_dim, int32_t group_size,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len,
                                int32_t causal, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */

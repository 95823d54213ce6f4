// Slot mapping and KV append (scatter into the paged pool).
//
// Address map: "3.3 Batching and memory management" (llm-learning-path),
// section "PagedAttention: the block table" -- token p of a sequence lives in
// physical block table[p / block_size] at offset p % block_size.  Append:
// "KV Cache: the memory bottleneck of LLM inference" (tag-page excerpt),
// section 1.1 -- the step's new k_t, v_t are written into the cache before
// attention reads it.
//
// Both kernels are tiny and latency bound (a decode step appends one token
// per sequence).  The append kernel moves whole 16-byte (or 8-byte for fp8
// output) pieces per lane so each row of head_dim elements is written with a
// handful of wide, coalesced stores.
#include "pa_device.h"

namespace pa {

// ---------------------------------------------------------------------------
// slot mapping: one workgroup per segment, lanes stride over its tokens
// ---------------------------------------------------------------------------
// Slot of logical position p through one sequence's table row, or -1 when p is
// negative, past the row, or its table entry is negative.
__device__ __forceinline__ int64_t map_slot(const int32_t* row, int max_blocks, int block_size,
                                            int64_t p) {
  const int64_t j = p / block_size;
  int64_t slot = -1;
  if (p >= 0 && j < max_blocks) {
    const int32_t blk = row[j];
    if (blk >= 0) slot = (int64_t)blk * block_size + (p - j * block_size);
  }
  return slot;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ tables, int max_blocks,
    int block_size, const int32_t* __restrict__ cu_tokens,
    const int32_t* __restrict__ start_pos) {
  const int s = blockIdx.x;
  const int t0 = cu_tokens[s], t1 = cu_tokens[s + 1];
  const int64_t p0 = start_pos[s];
  const int32_t* row = tables + (int64_t)s * max_blocks;
  for (int i = t0 + threadIdx.x; i < t1; i += blockDim.x)
    slots[i] = map_slot(row, max_blocks, block_size, p0 + (i - t0));
}

// The segment map of pa_slot_mapping, for the append kernels that compute each
// token's slot themselves (one launch instead of two).  Workgroup (s, y, kv)
// takes lane-pieces y*256 + tid, stepping by gridDim.y*256, of segment s's
// tokens; token indices are clamped to [0, num_tokens) so a malformed
// cu_tokens cannot reach past k_new / v_new.
struct SegMap {
  const int32_t* tables;
  const int32_t* cu_tokens;
  const int32_t* start_pos;
  int64_t* slots_out;   // optional: the slots, as pa_slot_mapping writes them
  int max_blocks;
  int block_size;
  int num_tokens;
};

struct SegRange {
  int t0, t1;
  int64_t p0;
  const int32_t* row;
};
__device__ __forceinline__ SegRange seg_range(const SegMap& m, int s) {
  SegRange r;
  r.t0 = max(0, uniform_load(m.cu_tokens, s));
  r.t1 = min(m.num_tokens, uniform_load(m.cu_tokens, s + 1));
  r.p0 = uniform_load(m.start_pos, s);
  r.row = m.tables + (int64_t)s * m.max_blocks;
  return r;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte read of source rows (read once, not kept in cache).
__device__ __forceinline__ uint4 ld_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int SRC, int DST>
struct AppendIO;

// Copies: 8 elements per lane.
template <>
struct AppendIO<PA_BF16, PA_BF16> {
  static __device__ __forceinline__ void run(const uint8_t* src, uint8_t* dst, float) {
    *(uint4*)dst = ld_stream(src);
  }
};
template <>
struct AppendIO<PA_F32, PA_F32> {
  static __device__ __forceinline__ void run(const uint8_t* src, uint8_t* dst, float) {
    const uint4 a = ld_stream(src);
    const uint4 b = ld_stream(src + 16);
    ((uint4*)dst)[0] = a;
    ((uint4*)dst)[1] = b;
  }
};
// Encodes (FP8_E4M3 or INT8): 8 elements in, 8 bytes out.
template <int DST>
struct AppendIO<PA_BF16, DST> {
  static __device__ __forceinline__ void run(const uint8_t* src, uint8_t* dst, float inv) {
    const uint4 a = ld_stream(src);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = encode8<DST>(bf16lo_f32(w[i]) * inv);
      const uint32_t hi = encode8<DST>(bf16hi_f32(w[i]) * inv);
      out[i >> 1] |= (lo | (hi << 8)) << ((i & 1) * 16);
    }
    *(uint2*)dst = make_uint2(out[0], out[1]);
  }
};
template <int DST>
struct AppendIO<PA_F32, DST> {
  static __device__ __forceinline__ void run(const uint8_t* src, uint8_t* dst, float inv) {
    const uint4 a = ld_stream(src);
    const uint4 b = ld_stream(src + 16);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i >> 2] |= encode8<DST>(bits_f32(w[i]) * inv) << ((i & 3) * 8);
    *(uint2*)dst = make_uint2(out[0], out[1]);
  }
};

constexpr int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : 1; }

// One lane moves 8 elements; a row (token, head) has head_dim / 8 lanes.
// grid.x covers num_tokens * n_kv * head_dim / 8 lanes for K, grid.y = 2 picks K or V.
// Piece `within` (8 elements) of token `tok`'s K or V row into slot `slot`.
template <int SRC, int DST>
__device__ __forceinline__ void append_piece(uint8_t* k_cache, uint8_t* v_cache,
                                             const uint8_t* k_new, const uint8_t* v_new,
                                             int64_t tok, int within, int64_t slot,
                                             int lanes_per_token, bool is_v, float inv) {
  constexpr int SB = elem_bytes(SRC), DB = elem_bytes(DST);
  const int64_t tok_elems = (int64_t)lanes_per_token * 8;  // n_kv * head_dim
  const uint8_t* src = (is_v ? v_new : k_new) + (tok * tok_elems + within * 8) * SB;
  uint8_t* dst = (is_v ? v_cache : k_cache) + (slot * tok_elems + within * 8) * DB;
  AppendIO<SRC, DST>::run(src, dst, inv);
}

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slots, int64_t num_slots_in_pool, int lanes_per_token,
    int total_lanes, float k_inv, float v_inv) {
  // 32-bit index arithmetic (the host keeps total_lanes below 2^31)
  const int lane = blockIdx.x * blockDim.x + threadIdx.x;
  if (lane >= total_lanes) return;
  const bool is_v = blockIdx.y != 0;
  const int tok = (int)((unsigned)lane / (unsigned)lanes_per_token);
  const int within = lane - tok * lanes_per_token;   // which 8-element piece of the token
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots_in_pool) return;
  append_piece<SRC, DST>(k_cache, v_cache, k_new, v_new, tok, within, slot, lanes_per_token, is_v,
                         is_v ? v_inv : k_inv);
}

// The same append with each token's slot computed from the block table.
template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_append_paged_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new, SegMap m,
    int64_t num_slots_in_pool, int lanes_per_token, float k_inv, float v_inv) {
  const SegRange r = seg_range(m, blockIdx.x);
  const bool is_v = blockIdx.z != 0;
  const int total = max(0, r.t1 - r.t0) * lanes_per_token;   // < 2^31 (host check)
  for (int L = blockIdx.y * 256 + threadIdx.x; L < total; L += gridDim.y * 256) {
    const int tl = (int)((unsigned)L / (unsigned)lanes_per_token);
    const int within = L - tl * lanes_per_token;
    const int64_t slot = map_slot(r.row, m.max_blocks, m.block_size, r.p0 + tl);
    if (!is_v && within == 0 && m.slots_out) m.slots_out[r.t0 + tl] = slot;
    if (slot < 0 || slot >= num_slots_in_pool) continue;
    append_piece<SRC, DST>(k_cache, v_cache, k_new, v_new, r.t0 + tl, within, slot,
                           lanes_per_token, is_v, is_v ? v_inv : k_inv);
  }
}

// ---------------------------------------------------------------------------
// INT4 append ("From PagedAttention to Chunked Prefill", section 5.4: KIVI's
// grouping -- keys quantised per channel, values per token).  Codes are
// symmetric in [-7, 7] (round half to even, clamp, NaN -> 0), two per byte in
// sign-magnitude nibbles, element 2i in the low nibble.  A key element is
// encoded with its channel's scale (k_channel_scales[head][dim], from the
// caller); a value row (token, head) gets the scale sigma = amax / 7 of its
// own elements (NaN ignored), stored in v_scales[block][head][offset].
//
// One row is head_dim / 8 lanes of 8 elements each (16 lanes at head_dim 128);
// the lanes of a value row find its amax with shuffles inside the row's lane
// group.  grid.y picks K or V.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_int4_nibble(float x) {
  if (!(x == x)) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(x, -7.0f), 7.0f));
  const int c = (int)r;
  return c < 0 ? 8u | (uint32_t)(-c) : (uint32_t)c;
}

template <int SRC>
__device__ __forceinline__ void load8_f32(const uint8_t* src, float (&x)[8]) {
  if constexpr (SRC == PA_BF16) {
    const uint4 a = ld_stream(src);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16lo_f32(w[i]); x[2 * i + 1] = bf16hi_f32(w[i]); }
  } else {
    const uint4 a = ld_stream(src), b = ld_stream(src + 16);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bits_f32(w[i]);
  }
}

// Piece j (8 elements) of row `row` (token * n_kv + head) into slot `slot`;
// every lane of the row's lane group must call it (the value rows' amax is
// found with shuffles inside the group), `ok` false only suppressing stores.
template <int SRC>
__device__ __forceinline__ void append_int4_piece(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, float* __restrict__ v_scales,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const float* __restrict__ k_channel_scales, int64_t row, int head, int j, int64_t slot,
    bool ok, int block_size, int n_kv, int lanes_per_row, bool is_v) {
  const int hd = lanes_per_row * 8;
  constexpr int SB = SRC == PA_F32 ? 4 : 2;
  float x[8];
  load8_f32<SRC>((is_v ? v_new : k_new) + ((int64_t)row * hd + j * 8) * SB, x);
  float inv[8];
  if (!is_v) {
    const float* sc = k_channel_scales + (int64_t)head * hd + j * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) inv[i] = 1.0f / sc[i];   // one binary32 division each
  } else {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));   // fmaxf ignores NaN
    for (int off = 1; off < lanes_per_row; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const float sigma = a / 7.0f;
    const float r = 1.0f / sigma;
#pragma unroll
    for (int i = 0; i < 8; ++i) inv[i] = r;
    if (ok && j == 0)   // [block][head][offset]
      v_scales[((slot / block_size) * n_kv + head) * block_size + slot % block_size] = sigma;
  }
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= f32_to_int4_nibble(x[i] * inv[i]) << (4 * i);
  if (ok) *(uint32_t*)((is_v ? v_cache : k_cache) + (slot * n_kv + head) * (hd / 2) + j * 4) = packed;
}

template <int SRC>
__global__ __launch_bounds__(256) void kv_append_int4_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, float* __restrict__ v_scales,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slots, const float* __restrict__ k_channel_scales,
    int64_t num_slots_in_pool, int block_size, int n_kv, int lanes_per_row, int total_lanes) {
  const int lane = blockIdx.x * blockDim.x + threadIdx.x;
  // every lane of a row takes part in the row's shuffles: no early return
  // before them (rows never straddle a wave: lanes_per_row divides 64)
  // idle lanes past the last row redo the last lane's reads (stores off), so
  // every load address stays inside k_new / v_new / k_channel_scales
  const bool live = lane < total_lanes;
  const int lc = min(lane, total_lanes - 1);
  const int row = (int)((unsigned)lc / (unsigned)lanes_per_row);
  const int j = lc - row * lanes_per_row;            // 8-element piece of the row
  const int tok = row / n_kv, head = row - tok * n_kv;
  const int64_t slot = slots[tok];
  const bool ok = live && slot >= 0 && slot < num_slots_in_pool;
  append_int4_piece<SRC>(k_cache, v_cache, v_scales, k_new, v_new, k_channel_scales, row, head, j,
                         slot, ok, block_size, n_kv, lanes_per_row, blockIdx.y != 0);
}

// The same append with each token's slot computed from the block table.  The
// loop bound is uniform over the workgroup, so every lane reaches the
// shuffles; rows never straddle a wave (256-lane strides, lanes_per_row
// divides 64).
template <int SRC>
__global__ __launch_bounds__(256) void kv_append_int4_paged_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, float* __restrict__ v_scales,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new, SegMap m,
    const float* __restrict__ k_channel_scales, int64_t num_slots_in_pool, int block_size,
    int n_kv, int lanes_per_row) {
  const SegRange r = seg_range(m, blockIdx.x);
  const bool is_v = blockIdx.z != 0;
  const int total = max(0, r.t1 - r.t0) * n_kv * lanes_per_row;   // < 2^31 (host check)
  for (int base = blockIdx.y * 256; base < total; base += gridDim.y * 256) {
    const int L = base + threadIdx.x;
    const bool live = L < total;
    const int rl = (int)((unsigned)min(L, total - 1) / (unsigned)lanes_per_row);
    const int j = min(L, total - 1) - rl * lanes_per_row;
    const int tl = rl / n_kv, head = rl - tl * n_kv;
    const int64_t slot = map_slot(r.row, m.max_blocks, m.block_size, r.p0 + tl);
    if (!is_v && live && j == 0 && head == 0 && m.slots_out) m.slots_out[r.t0 + tl] = slot;
    const bool ok = live && slot >= 0 && slot < num_slots_in_pool;
    append_int4_piece<SRC>(k_cache, v_cache, v_scales, k_new, v_new, k_channel_scales,
                           (int64_t)(r.t0 + tl) * n_kv + head, head, j, slot, ok, block_size, n_kv,
                           lanes_per_row, is_v);
  }
}

}  // namespace pa

using namespace pa;

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent or negative sizes";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unsupported dtype or dtype pair";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim/block_size/group_size not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch or runtime call failed";
    default: return "PA_ERR_UNKNOWN";
  }
}

extern "C" int pa_abi_version(void) { return 2; }

extern "C" pa_status pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, int32_t block_size,
                                     const int32_t* cu_tokens, const int32_t* start_pos,
                                     int32_t num_seqs, int32_t num_tokens, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || block_size < 1 || max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!slot_mapping || !block_tables || !cu_tokens || !start_pos) return PA_ERR_NULL;
  return launch(slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, (hipStream_t)stream,
                     slot_mapping, block_tables, max_blocks_per_seq, block_size, cu_tokens,
                     start_pos);
}

extern "C" pa_status pa_kv_append(void* k_cache, void* v_cache, int cache_dtype,
                                  int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                  int32_t head_dim, const void* k_new, const void* v_new,
                                  int src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                                  float k_scale, float v_scale, void* stream) {
  if (num_blocks < 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || num_tokens < 0)
    return PA_ERR_SHAPE;
  if (head_dim % 8 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  const int64_t lanes = (int64_t)n_kv_heads * head_dim / 8;
  if (lanes * num_tokens >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  const int lanes_per_token = (int)lanes;
  const int total = (int)(lanes * num_tokens);
  const int64_t pool_slots = (int64_t)num_blocks * block_size;
  const dim3 grid((unsigned)((total + 255) / 256), 2);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* kc = (uint8_t*)k_cache;
  uint8_t* vc = (uint8_t*)v_cache;
  const uint8_t* kn = (const uint8_t*)k_new;
  const uint8_t* vn = (const uint8_t*)v_new;
  if (cache_dtype == src_dtype && cache_dtype == PA_BF16) {
    return launch((kv_append_kernel<PA_BF16, PA_BF16>), grid, dim3(256), 0, st, kc, vc, kn,
                       vn, slot_mapping, pool_slots, lanes_per_token, total, 1.0f, 1.0f);
  } else if (cache_dtype == src_dtype && cache_dtype == PA_F32) {
    return launch((kv_append_kernel<PA_F32, PA_F32>), grid, dim3(256), 0, st, kc, vc, kn,
                       vn, slot_mapping, pool_slots, lanes_per_token, total, 1.0f, 1.0f);
  } else if ((cache_dtype == PA_FP8_E4M3 || cache_dtype == PA_INT8) &&
             (src_dtype == PA_BF16 || src_dtype == PA_F32)) {
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f)) return PA_ERR_SHAPE;
    const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;   // one binary32 division each
    const bool i8 = cache_dtype == PA_INT8;
    auto kernel = src_dtype == PA_BF16 ? (i8 ? kv_append_kernel<PA_BF16, PA_INT8>
                                             : kv_append_kernel<PA_BF16, PA_FP8_E4M3>)
                                       : (i8 ? kv_append_kernel<PA_F32, PA_INT8>
                                             : kv_append_kernel<PA_F32, PA_FP8_E4M3>);
    return launch(kernel, grid, dim3(256), 0, st, kc, vc, kn, vn, slot_mapping, pool_slots,
                       lanes_per_token, total, k_inv, v_inv);
  }
  return PA_ERR_DTYPE;
}

extern "C" pa_status pa_kv_append_int4(void* k_cache, void* v_cache, float* v_scales,
                                       int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                                       int32_t head_dim, const void* k_new, const void* v_new,
                                       int src_dtype, const int64_t* slot_mapping,
                                       int32_t num_tokens, const float* k_channel_scales,
                                       void* stream) {
  if (num_blocks < 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || num_tokens < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (src_dtype != PA_BF16 && src_dtype != PA_F32) return PA_ERR_DTYPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !v_scales || !k_new || !v_new || !slot_mapping || !k_channel_scales)
    return PA_ERR_NULL;
  const int lanes_per_row = head_dim / 8;
  const int64_t lanes = (int64_t)num_tokens * n_kv_heads * lanes_per_row;
  if (lanes >= ((int64_t)1 << 31) - 256) return PA_ERR_SHAPE;
  const int total = (int)lanes;
  const dim3 grid((unsigned)((total + 255) / 256), 2);
  auto kernel = src_dtype == PA_BF16 ? kv_append_int4_kernel<PA_BF16> : kv_append_int4_kernel<PA_F32>;
  return launch(kernel, grid, dim3(256), 0, (hipStream_t)stream, (uint8_t*)k_cache,
                     (uint8_t*)v_cache, v_scales, (const uint8_t*)k_new, (const uint8_t*)v_new,
                     slot_mapping, k_channel_scales, (int64_t)num_blocks * block_size, block_size,
                     n_kv_heads, lanes_per_row, total);
}

// Grid of the paged appends: one workgroup row per segment, enough 256-lane
// workgroups per segment for max_tokens_per_seq tokens (a hint: longer
// segments loop), K and V in grid.z.
static dim3 paged_grid(int num_seqs, int max_tokens_per_seq, int64_t lanes_per_token) {
  int64_t gy = ((int64_t)max(1, max_tokens_per_seq) * lanes_per_token + 255) / 256;
  if (gy > 65535) gy = 65535;
  return dim3((unsigned)num_seqs, (unsigned)gy, 2);
}

extern "C" pa_status pa_kv_append_paged(void* k_cache, void* v_cache, int cache_dtype,
                                        int32_t num_blocks, int32_t block_size,
                                        int32_t n_kv_heads, int32_t head_dim, const void* k_new,
                                        const void* v_new, int src_dtype,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* cu_tokens, const int32_t* start_pos,
                                        int32_t num_seqs, int32_t num_tokens,
                                        int32_t max_tokens_per_seq, int64_t* slot_mapping,
                                        float k_scale, float v_scale, void* stream) {
  if (num_blocks < 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || num_tokens < 0 ||
      num_seqs < 0 || max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (head_dim % 8 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0 || num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !cu_tokens || !start_pos)
    return PA_ERR_NULL;
  const int64_t lanes = (int64_t)n_kv_heads * head_dim / 8;
  if (lanes * num_tokens >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  SegMap m;
  m.tables = block_tables; m.cu_tokens = cu_tokens; m.start_pos = start_pos;
  m.slots_out = slot_mapping; m.max_blocks = max_blocks_per_seq; m.block_size = block_size;
  m.num_tokens = num_tokens;
  const int64_t pool_slots = (int64_t)num_blocks * block_size;
  const dim3 grid = paged_grid(num_seqs, max_tokens_per_seq, lanes);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* kc = (uint8_t*)k_cache;
  uint8_t* vc = (uint8_t*)v_cache;
  const uint8_t* kn = (const uint8_t*)k_new;
  const uint8_t* vn = (const uint8_t*)v_new;
  const int lpt = (int)lanes;
  if (cache_dtype == src_dtype && cache_dtype == PA_BF16) {
    return launch((kv_append_paged_kernel<PA_BF16, PA_BF16>), grid, dim3(256), 0, st, kc, vc,
                       kn, vn, m, pool_slots, lpt, 1.0f, 1.0f);
  } else if (cache_dtype == src_dtype && cache_dtype == PA_F32) {
    return launch((kv_append_paged_kernel<PA_F32, PA_F32>), grid, dim3(256), 0, st, kc, vc,
                       kn, vn, m, pool_slots, lpt, 1.0f, 1.0f);
  } else if ((cache_dtype == PA_FP8_E4M3 || cache_dtype == PA_INT8) &&
             (src_dtype == PA_BF16 || src_dtype == PA_F32)) {
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f)) return PA_ERR_SHAPE;
    const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;   // one binary32 division each
    const bool i8 = cache_dtype == PA_INT8;
    auto kernel = src_dtype == PA_BF16
                      ? (i8 ? kv_append_paged_kernel<PA_BF16, PA_INT8>
                            : kv_append_paged_kernel<PA_BF16, PA_FP8_E4M3>)
                      : (i8 ? kv_append_paged_kernel<PA_F32, PA_INT8>
                            : kv_append_paged_kernel<PA_F32, PA_FP8_E4M3>);
    return launch(kernel, grid, dim3(256), 0, st, kc, vc, kn, vn, m, pool_slots, lpt, k_inv,
                       v_inv);
  }
  return PA_ERR_DTYPE;
}

extern "C" pa_status pa_kv_append_int4_paged(void* k_cache, void* v_cache, float* v_scales,
                                             int32_t num_blocks, int32_t block_size,
                                             int32_t n_kv_heads, int32_t head_dim,
                                             const void* k_new, const void* v_new, int src_dtype,
                                             const int32_t* block_tables,
                                             int32_t max_blocks_per_seq, const int32_t* cu_tokens,
                                             const int32_t* start_pos, int32_t num_seqs,
                                             int32_t num_tokens, int32_t max_tokens_per_seq,
                                             int64_t* slot_mapping,
                                             const float* k_channel_scales, void* stream) {
  if (num_blocks < 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || num_tokens < 0 ||
      num_seqs < 0 || max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (src_dtype != PA_BF16 && src_dtype != PA_F32) return PA_ERR_DTYPE;
  if (num_tokens == 0 || num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !v_scales || !k_new || !v_new || !block_tables || !cu_tokens ||
      !start_pos || !k_channel_scales)
    return PA_ERR_NULL;
  const int lanes_per_row = head_dim / 8;
  const int64_t lanes = (int64_t)n_kv_heads * lanes_per_row;
  if (lanes * num_tokens >= ((int64_t)1 << 31) - 256) return PA_ERR_SHAPE;
  SegMap m;
  m.tables = block_tables; m.cu_tokens = cu_tokens; m.start_pos = start_pos;
  m.slots_out = slot_mapping; m.max_blocks = max_blocks_per_seq; m.block_size = block_size;
  m.num_tokens = num_tokens;
  const dim3 grid = paged_grid(num_seqs, max_tokens_per_seq, lanes);
  auto kernel = src_dtype == PA_BF16 ? kv_append_int4_paged_kernel<PA_BF16>
                                     : kv_append_int4_paged_kernel<PA_F32>;
  return launch(kernel, grid, dim3(256), 0, (hipStream_t)stream, (uint8_t*)k_cache,
                     (uint8_t*)v_cache, v_scales, (const uint8_t*)k_new, (const uint8_t*)v_new, m,
                     k_channel_scales, (int64_t)num_blocks * block_size, block_size, n_kv_heads,
                     lanes_per_row);
}

// Whole-block copies between paged pools.
//
// "3.3 Batching and memory management", section "Sharing and copy-on-write":
// a block still referenced by other sequences is copied to a fresh block
// before one of them writes into it; section "Scheduling policy and
// preemption": a preempted sequence's blocks are copied out to host memory
// and copied back (to whatever blocks are free) when it resumes.  Both are a
// list of (source block, destination block) pairs applied to K and V: within
// one device pool, or between a device pool and a pool in pinned host memory
// (which the kernel reads or writes directly over the host link).
//
// The copy is bandwidth bound: each workgroup moves one 16 KiB chunk of one
// block of K or V with 16-byte (8-byte when the block size needs it) loads and
// stores, all of a lane's loads issued before its stores, so a batch of pairs
// spreads over the whole chip with many reads in flight.  The loads are
// non-temporal (the source is read once); the stores are ordinary: measured
// on 4096 Llama-3 block pairs, 6.3 TB/s of reads plus writes against 5.0 TB/s
// with non-temporal stores (and 5.4 TB/s for hipMemcpyAsync of the same bytes
// as one contiguous device-to-device copy).
#include "pa_device.h"

namespace pa {

constexpr int CB_THREADS = 256;
constexpr int64_t CB_CHUNK = 16384;   // bytes of a block per workgroup

template <int VEC>
struct CopyVec;
template <>
struct CopyVec<16> {
  typedef uint32_t T __attribute__((ext_vector_type(4)));
};
template <>
struct CopyVec<8> {
  typedef uint32_t T __attribute__((ext_vector_type(2)));
};

template <int VEC>
__global__ __launch_bounds__(CB_THREADS) void copy_blocks_kernel(
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, int64_t dst_blocks,
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v, int64_t src_blocks,
    const int64_t* __restrict__ pairs, int64_t block_bytes, int chunks_per_block) {
  typedef typename CopyVec<VEC>::T V;
  // every load of the chunk is issued before the first store, so a lane keeps
  // CB_CHUNK / (CB_THREADS * VEC) loads in flight instead of one
  constexpr int N = (int)(CB_CHUNK / (CB_THREADS * VEC));
  const int pair = blockIdx.x / chunks_per_block;
  const int chunk = blockIdx.x % chunks_per_block;
  const int64_t s = pairs[2 * (int64_t)pair], d = pairs[2 * (int64_t)pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const uint8_t* src = (blockIdx.y ? src_v : src_k) + s * block_bytes;
  uint8_t* dst = (blockIdx.y ? dst_v : dst_k) + d * block_bytes;
  const int64_t base = (int64_t)chunk * CB_CHUNK + threadIdx.x * VEC;
  const int64_t end = min(block_bytes, (int64_t)(chunk + 1) * CB_CHUNK);
  V x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int64_t off = base + (int64_t)i * CB_THREADS * VEC;
    if (off < end) x[i] = __builtin_nontemporal_load((const V*)(src + off));
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int64_t off = base + (int64_t)i * CB_THREADS * VEC;
    if (off < end) *(V*)(dst + off) = x[i];
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_copy_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks,
                                    const void* src_k, const void* src_v, int32_t src_num_blocks,
                                    int cache_dtype, int32_t block_size, int32_t n_kv_heads,
                                    int32_t head_dim, const int64_t* block_pairs,
                                    int32_t num_pairs, void* stream) {
  if (dst_num_blocks < 0 || src_num_blocks < 0 || block_size < 1 || n_kv_heads < 1 ||
      head_dim < 1 || num_pairs < 0)
    return PA_ERR_SHAPE;
  if (cache_dtype != PA_F32 && cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3 &&
      cache_dtype != PA_INT8 && cache_dtype != PA_INT4)
    return PA_ERR_DTYPE;
  const int ebits = cache_dtype == PA_F32 ? 32 : cache_dtype == PA_BF16 ? 16
                  : cache_dtype == PA_INT4 ? 4 : 8;
  const int64_t block_bytes = (int64_t)block_size * n_kv_heads * head_dim * ebits / 8;
  if (block_bytes % 8) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PA_ERR_NULL;
  const int vec = block_bytes % 16 == 0 ? 16 : 8;
  for (const void* p : {(const void*)dst_k, (const void*)dst_v, src_k, src_v})
    if ((uintptr_t)p % vec) return PA_ERR_SHAPE;
  const int64_t chunks = (block_bytes + CB_CHUNK - 1) / CB_CHUNK;
  if ((int64_t)num_pairs * chunks >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  const dim3 grid((unsigned)(num_pairs * chunks), 2);
  hipStream_t st = (hipStream_t)stream;
  if (vec == 16)
    return launch(copy_blocks_kernel<16>, grid, dim3(CB_THREADS), 0, st, (uint8_t*)dst_k,
                  (uint8_t*)dst_v, (int64_t)dst_num_blocks, (const uint8_t*)src_k,
                  (const uint8_t*)src_v, (int64_t)src_num_blocks, block_pairs, block_bytes,
                  (int)chunks);
  return launch(copy_blocks_kernel<8>, grid, dim3(CB_THREADS), 0, st, (uint8_t*)dst_k,
                (uint8_t*)dst_v, (int64_t)dst_num_blocks, (const uint8_t*)src_k,
                (const uint8_t*)src_v, (int64_t)src_num_blocks, block_pairs, block_bytes,
                (int)chunks);
}

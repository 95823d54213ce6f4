// Measured ceilings of the device: what a kernel that only reads whole pool
// blocks, or only issues matrix-core instructions, reaches on this GPU.  They
// are the yardsticks the benchmark reports beside the published peaks (8 TB/s
// HBM, 2.5 PFLOP/s dense bf16): a decode kernel is judged against what reading
// the same blocks in the same order can reach (and in physical order, for the
// cost of the order), the prefill kernel against what v_mfma_f32_32x32x16_bf16
// can reach, with its operands in registers and with one operand read from LDS
// for every instruction, as the prefill kernel reads K and V^T.  Not part of the attention path: built into libpa_probes.so, a
// library of its own that only the benchmark and its tests load.
//
// Every reader folds what it reads into an XOR checksum that it writes out, so
// the loads cannot be dropped and a test can check that exactly the intended
// bytes were read.
#include "../csrc/pa_device.h"
#include "pa_probes.h"

namespace pa {

typedef uint32_t cu32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ cu32x4_t ld_nt16(const uint8_t* p) {
  return __builtin_nontemporal_load((const cu32x4_t*)p);
}

// One XOR per wave, no workgroup barrier: sink[workgroup * 4 + wave].
__device__ __forceinline__ void reduce_xor_store(uint32_t x, uint32_t* sink) {
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

// Contiguous read of `chunks` 16-byte chunks: workgroup w reads an equal
// contiguous share, 8 loads in flight per lane.
__global__ __launch_bounds__(256) void ceiling_stream_kernel(const uint8_t* __restrict__ buf,
                                                             int64_t chunks, uint32_t* sink) {
  const int64_t W = gridDim.x;
  const int64_t c0 = (int64_t)blockIdx.x * chunks / W, c1 = (int64_t)(blockIdx.x + 1) * chunks / W;
  uint32_t x = 0;
  int64_t c = c0 + threadIdx.x;
  for (; c + 7 * 256 < c1; c += 8 * 256) {
    cu32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld_nt16(buf + 16 * (c + 256 * u));
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; c < c1; c += 256) {
    const cu32x4_t a = ld_nt16(buf + 16 * c);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  reduce_xor_store(x, sink);
}

// Whole blocks of two pools in list order: entry i of `blocks` names a block
// of `block_bytes` bytes in k_pool and the same block in v_pool.  Workgroup w
// reads an equal contiguous share of the list, each block as one run of
// 16-byte loads (the order a paged decode reads its blocks in).
__global__ __launch_bounds__(256) void ceiling_gather_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    const int32_t* __restrict__ blocks, int64_t n, int64_t pool_blocks, int block_bytes,
    uint32_t* sink) {
  const int64_t W = gridDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * n / W, i1 = (int64_t)(blockIdx.x + 1) * n / W;
  const int per = block_bytes / 16;   // chunks per block
  uint32_t x = 0;
  // the next block id is read while the current block streams in
  int nxt = i0 < i1 ? uniform_load(blocks, (int)i0) : 0;
  for (int64_t i = i0; i < i1; ++i) {
    int blk = nxt;
    nxt = uniform_load(blocks, (int)min(i + 1, i1 - 1));
    blk = (uint64_t)(uint32_t)blk < (uint64_t)pool_blocks ? blk : 0;
    const int64_t off = (int64_t)blk * block_bytes;
#pragma unroll 8
    for (int c = threadIdx.x; c < per; c += 256) {
      const cu32x4_t a = ld_nt16(k_pool + off + 16 * c), b = ld_nt16(v_pool + off + 16 * c);
      x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    }
  }
  reduce_xor_store(x, sink);
}

// Matrix-core issue rate: every wave runs `iters` rounds of 4 independent
// v_mfma_f32_32x32x16_bf16 chains on register operands (A = B = 1.0), so each
// accumulator element ends at 16 * iters.
typedef __bf16 cbf16x8_t __attribute__((ext_vector_type(8)));
typedef float cf32x16_t __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void ceiling_mfma_kernel(int iters, float* sink) {
  cbf16x8_t one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = (__bf16)1.0f;
  cf32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  // every lane's sum is 64 * 16 * iters; one value per wave
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

}  // namespace pa

using namespace pa;

// The prefill kernel's operand traffic without its softmax: every MFMA reads its
// A operand (32 rows x 16 bf16, 1 KiB per wave) from LDS with one ds_read_b128
// per lane, as the score (K) and PV (V^T) products do; B stays in registers.
// Each wave cycles through 16 KiB of LDS, 1 KiB per read, consecutive lanes on
// consecutive 16-byte chunks (no bank conflicts).
constexpr int CEIL_LDS_BYTES = 16 * 1024;
__global__ __launch_bounds__(256) void ceiling_mfma_lds_kernel(int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[CEIL_LDS_BYTES];
  for (int i = threadIdx.x; i < CEIL_LDS_BYTES / 4; i += blockDim.x)
    ((uint32_t*)lds)[i] = 0x3F803F80u;   // bf16 pairs of 1.0
  __syncthreads();
  cbf16x8_t one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = (__bf16)1.0f;
  cf32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < iters; ++i) {
    const int base = ((4 * i) & 15) * 1024 + lane * 16;
    const cbf16x8_t a0 = *(const cbf16x8_t*)(lds + base);
    const cbf16x8_t a1 = *(const cbf16x8_t*)(lds + ((base + 1024) & (CEIL_LDS_BYTES - 1)));
    const cbf16x8_t a2 = *(const cbf16x8_t*)(lds + ((base + 2048) & (CEIL_LDS_BYTES - 1)));
    const cbf16x8_t a3 = *(const cbf16x8_t*)(lds + ((base + 3072) & (CEIL_LDS_BYTES - 1)));
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, one, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, one, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, one, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, one, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

extern "C" pa_status pa_ceiling_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                            int32_t num_wgs, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || num_wgs < 1) return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return PA_ERR_NULL;
  return launch(ceiling_stream_kernel, dim3((unsigned)num_wgs), dim3(256), 0, (hipStream_t)stream,
                (const uint8_t*)buf, bytes / 16, sink);
}

extern "C" pa_status pa_ceiling_gather_read(const void* k_pool, const void* v_pool,
                                            int64_t pool_blocks, int32_t block_bytes,
                                            const int32_t* blocks, int64_t n, uint32_t* sink,
                                            int32_t num_wgs, void* stream) {
  if (n < 0 || block_bytes < 16 || block_bytes % 16 != 0 || num_wgs < 1 || pool_blocks < 0 ||
      n > 2147483647)
    return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !blocks || !sink) return PA_ERR_NULL;
  if (pool_blocks == 0) return PA_ERR_SHAPE;
  // entries outside [0, pool_blocks) read block 0
  return launch(ceiling_gather_kernel, dim3((unsigned)num_wgs), dim3(256), 0, (hipStream_t)stream,
                (const uint8_t*)k_pool, (const uint8_t*)v_pool, blocks, n, pool_blocks,
                block_bytes, sink);
}

extern "C" pa_status pa_ceiling_mfma_bf16(float* sink, int32_t num_wgs, int32_t iters,
                                          void* stream) {
  if (num_wgs < 1 || iters < 1) return PA_ERR_SHAPE;
  if (!sink) return PA_ERR_NULL;
  return launch(ceiling_mfma_kernel, dim3((unsigned)num_wgs), dim3(256), 0, (hipStream_t)stream,
                iters, sink);
}

extern "C" pa_status pa_ceiling_mfma_bf16_lds(float* sink, int32_t num_wgs, int32_t iters,
                                              void* stream) {
  if (num_wgs < 1 || iters < 1) return PA_ERR_SHAPE;
  if (!sink) return PA_ERR_NULL;
  return launch(ceiling_mfma_lds_kernel, dim3((unsigned)num_wgs), dim3(256), 0,
                (hipStream_t)stream, iters, sink);
}

// LDS bank-group probe: one wave per workgroup repeats one LDS access, with a
// byte offset per lane taken from a table, so that the SQ_LDS_BANK_CONFLICT
// counter of each launch measures one access pattern.  The decode kernels'
// LDS swizzles (the load stage and the per-wave V slices) were chosen from
// these measurements.  Not part of the attention path (libpa_probes.so).
#include "../csrc/pa_device.h"
#include "pa_probes.h"

namespace pa {

constexpr int LP_BYTES = 16384;

typedef short lp_s4_t __attribute__((ext_vector_type(4)));

// 16-bit element k of the LDS area holds lp_fill(k); a read folds what it got
// into one XOR of 16-bit elements, which does not depend on how the
// transposing read spreads the elements over the lanes.
__device__ __forceinline__ uint32_t lp_fill(uint32_t k) { return (k * 40503u) & 0xffffu; }
__device__ __forceinline__ uint32_t lp_fold(uint32_t w) { return (w & 0xffffu) ^ (w >> 16); }

template <int KIND>
__global__ __launch_bounds__(64) void lds_pattern_kernel(const uint32_t* __restrict__ offsets,
                                                         int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LP_BYTES];
  const int lane = threadIdx.x;
  for (int i = lane; i < LP_BYTES / 4; i += 64) {
    const uint32_t k = 2u * (uint32_t)i;
    *(uint32_t*)(lds + 4 * i) = lp_fill(k) | (lp_fill(k + 1) << 16);
  }
  __syncthreads();
  // clamped and aligned into the area, so every access stays inside it
  constexpr uint32_t SIZE = KIND >= 2 ? 8u : 16u;
  const uint32_t off = min(offsets[lane], (uint32_t)LP_BYTES - SIZE) & ~(SIZE - 1u);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0) {          // ds_write_b128
      *(uint4*)(lds + off) = make_uint4((uint32_t)it, acc, (uint32_t)lane, 0u);
    } else if constexpr (KIND == 1) {   // ds_read_b128
      const uint4 v = *(const uint4*)(lds + off);
      acc ^= lp_fold(v.x) ^ lp_fold(v.y) ^ lp_fold(v.z) ^ lp_fold(v.w);
    } else if constexpr (KIND == 2) {   // ds_read_b64_tr_b16
      const lp_s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) lp_s4_t*)(lds + off));
      acc ^= (uint32_t)(uint16_t)v[0] ^ (uint32_t)(uint16_t)v[1] ^ (uint32_t)(uint16_t)v[2] ^
             (uint32_t)(uint16_t)v[3];
    } else {                            // ds_read_b64
      const uint2 v = *(const uint2*)(lds + off);
      acc ^= lp_fold(v.x) ^ lp_fold(v.y);
    }
    asm volatile("" ::: "memory");
  }
  for (int s = 32; s > 0; s >>= 1) acc ^= __shfl_xor(acc, s, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_probe_lds_pattern(const uint32_t* offsets, int32_t kind, int32_t iters,
                                          uint32_t* sink, int32_t num_wgs, void* stream) {
  if (kind < 0 || kind > 3 || iters < 1 || num_wgs < 1) return PA_ERR_SHAPE;
  if (!offsets || !sink) return PA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const dim3 g((unsigned)num_wgs), b(64);
  switch (kind) {
    case 0: return launch(lds_pattern_kernel<0>, g, b, 0, st, offsets, iters, sink);
    case 1: return launch(lds_pattern_kernel<1>, g, b, 0, st, offsets, iters, sink);
    case 2: return launch(lds_pattern_kernel<2>, g, b, 0, st, offsets, iters, sink);
    default: return launch(lds_pattern_kernel<3>, g, b, 0, st, offsets, iters, sink);
  }
}

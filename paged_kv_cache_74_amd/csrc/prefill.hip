// Chunked-prefill attention over the paged KV cache, on MFMA.
//
// What is computed:
//   * a chunk of L query tokens of a sequence whose cache already holds the
//     earlier tokens and the chunk's own K/V (appended first) attends to that
//     cache -- "3.3 Batching and memory management", section "Chunked
//     prefill"; query i of the chunk sits at position T - L + i (T = context
//     length including the chunk) and, with the causal mask, sees keys j <= it;
//   * the batch is ragged: chunk s owns query rows [cu_seqlens_q[s],
//     cu_seqlens_q[s+1]) -- "From PagedAttention to Chunked Prefill", section
//     3.2 (mixed query lengths located by cumulative offsets);
//   * K/V gathered through the block table (token p in block
//     table[p / block_size] at offset p % block_size -- "PagedAttention: the
//     block table"), softmax accumulated tile by tile with the online
//     recurrence ("From PagedAttention to Chunked Prefill", section 2.2).
//
// How it maps to CDNA4 (gfx950):
//   * A workgroup of 4 waves owns 128 query rows: the group_size query heads of
//     one KV head times 128 / group_size consecutive queries, so each K/V tile
//     staged in LDS serves every head of the group.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K rows (A operand) and Q rows (B operand) are both read along head_dim,
//     their natural layout.  In the result each lane holds 16 keys of one
//     query row, so the row max needs one exchange with lane l ^ 32.
//   * O^T = V^T P^T: the probability registers of the score tile are already
//     the B operand of the PV MFMA (the key order inside a 16-key slice is
//     permuted consistently in both operands); only V is stored transposed in
//     LDS, written as bf16 pairs of two keys.
//   * Rows are rescaled only when some row's running max grew (wave-uniform).
#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int PF_WAVES = 4;
constexpr int PF_ROWS = 32 * PF_WAVES;   // query rows per workgroup
constexpr int PF_BN = 32;                // keys per tile

struct PrefillArgs {
  const uint8_t* q;          // [total_q][n_q][HD] bf16
  void* out;                 // [total_q][n_q][HD] bf16
  const int32_t* cu_q;       // [num_seqs + 1]
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t tok_stride;        // bytes between consecutive tokens of a block
  int num_blocks;
  int block_size;
  int bs_log2;
  int n_kv;
  int max_blocks;
  int qtiles;                // query tiles per sequence (grid bound)
  int causal;
  float score_scale;         // scale * k_scale * log2(e)
  float out_scale;           // v_scale for fp8 caches, else 1
};

template <int CDT, int HD>
struct PrefillLds {
  static constexpr int KROW = HD * 2 + 16;        // bytes per key row of K (padded)
  static constexpr int VROW = PF_BN * 2 + 16;     // bytes per dim row of V^T (padded)
  static constexpr int K_BYTES = PF_BN * KROW;
  static constexpr int V_BYTES = HD * VROW;
};

// Physical address of token `key` (kv head kvh, byte `col` of the row), or
// nullptr when the token is outside the context or its block id is invalid.
__device__ __forceinline__ const uint8_t* token_ptr(const uint8_t* cache, const PrefillArgs& a,
                                                    const int32_t* table, int key, int T, int kvh,
                                                    int row_bytes, int col) {
  if (key >= T) return nullptr;
  const int j = key >> a.bs_log2;
  if (j >= a.max_blocks) return nullptr;
  const int blk = table[j];
  if ((unsigned)blk >= (unsigned)a.num_blocks) return nullptr;
  return cache + ((int64_t)blk * a.block_size + (key & (a.block_size - 1))) * a.tok_stride +
         (int64_t)kvh * row_bytes + col;
}

// 8 cache elements of one token row -> 4 dwords of bf16 pairs
template <int CDT>
__device__ __forceinline__ void load8(const uint8_t* p, uint32_t (&d)[4]) {
  if (!p) { d[0] = d[1] = d[2] = d[3] = 0u; return; }
  if constexpr (CDT == PA_BF16) {
    const uint4 x = *(const uint4*)p;
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
  } else {   // fp8 e4m3: 8 bytes -> 4 bf16 pairs (exact)
    const uint2 x = *(const uint2*)p;
    d[0] = fp8x2_to_bf16x2<false>(x.x); d[1] = fp8x2_to_bf16x2<true>(x.x);
    d[2] = fp8x2_to_bf16x2<false>(x.y); d[3] = fp8x2_to_bf16x2<true>(x.y);
  }
}

template <int CDT, int HD, int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  using LD = PrefillLds<CDT, HD>;
  constexpr int QB = PF_ROWS / G;            // queries per workgroup
  constexpr int EB = CDT == PA_BF16 ? 2 : 1;
  constexpr int ROWB = HD * EB;              // bytes of one (token, head) row in the cache
  constexpr int NDT = HD / 32;               // 32-dim output tiles
  constexpr int NKT = HD / 16;               // 16-dim steps of the score MFMA
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[LD::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[LD::V_BYTES];

  int wid = blockIdx.x;
  const int kvh = wid % a.n_kv;
  wid /= a.n_kv;
  const int qtile = wid % a.qtiles;
  const int s = wid / a.qtiles;
  const int q0 = a.cu_q[s];
  const int L = a.cu_q[s + 1] - q0;
  if (qtile * QB >= L) return;
  const int T = a.context_lens[s];
  const int n_q = a.n_kv * G;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, grp = lane >> 5;
  // this lane's query row
  const int rr = wave * 32 + lr;
  const int hl = rr / QB;
  const int qi = qtile * QB + rr % QB;
  const bool row_ok = qi < L;
  const int pos = T - L + qi;
  const int head = kvh * G + hl;

  // Q operand: Q[row][16t + 8 grp + e]
  uint32_t qreg[NKT][4];
  {
    const uint8_t* qp = a.q + ((int64_t)(q0 + qi) * n_q + head) * HD * 2 + grp * 16;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      if (row_ok) {
        const uint4 x = *(const uint4*)(qp + t * 32);
        qreg[t][0] = x.x; qreg[t][1] = x.y; qreg[t][2] = x.z; qreg[t][3] = x.w;
      } else {
        qreg[t][0] = qreg[t][1] = qreg[t][2] = qreg[t][3] = 0u;
      }
    }
  }

  // keys this workgroup needs
  const int last_q = min(L, (qtile + 1) * QB) - 1;
  const int first_pos = T - L + qtile * QB;
  const int visible = a.causal ? min(T, T - L + last_q + 1) : T;
  const int n_tiles = (visible + PF_BN - 1) / PF_BN;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;

  f32x16_t acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
  float m = -1e30f, lsum = 0.0f;
  const float c = a.score_scale;

  // cooperative tile load: thread -> (key pair, 8-element chunk of the row)
  constexpr int CHUNKS = HD / 8;
  const int lp = tid / CHUNKS;               // key pair 0..15 (valid when < 16)
  const int lc = tid % CHUNKS;
  const bool loader = lp < PF_BN / 2;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int kb = kt * PF_BN;
    if (loader) {
      uint32_t k0[4], k1[4], v0[4], v1[4];
      const int key0 = kb + 2 * lp;
      load8<CDT>(token_ptr(a.k_cache, a, table, key0, T, kvh, ROWB, lc * 8 * EB), k0);
      load8<CDT>(token_ptr(a.k_cache, a, table, key0 + 1, T, kvh, ROWB, lc * 8 * EB), k1);
      load8<CDT>(token_ptr(a.v_cache, a, table, key0, T, kvh, ROWB, lc * 8 * EB), v0);
      load8<CDT>(token_ptr(a.v_cache, a, table, key0 + 1, T, kvh, ROWB, lc * 8 * EB), v1);
      *(uint4*)(lds_k + (2 * lp) * LD::KROW + lc * 16) = make_uint4(k0[0], k0[1], k0[2], k0[3]);
      *(uint4*)(lds_k + (2 * lp + 1) * LD::KROW + lc * 16) = make_uint4(k1[0], k1[1], k1[2], k1[3]);
      // V^T[d][key0, key0 + 1] as one bf16 pair per dim
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lc * 8 + 2 * i;
        *(uint32_t*)(lds_v + d * LD::VROW + 4 * lp) = pair_lo(v0[i], v1[i]);
        *(uint32_t*)(lds_v + (d + 1) * LD::VROW + 4 * lp) = pair_hi(v0[i], v1[i]);
      }
    }
    __syncthreads();

    // S^T tile (32 keys x 32 rows of this wave)
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const uint4 kx = *(const uint4*)(lds_k + lr * LD::KROW + (16 * t + 8 * grp) * 2);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, kx);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(qreg[t][0], qreg[t][1], qreg[t][2], qreg[t][3]));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, sc, 0, 0, 0);
    }
    // mask (ragged end, causal diagonal) and scale into the log2 domain
    const bool full_tile = kb + PF_BN <= T && (!a.causal || kb + PF_BN - 1 <= first_pos);
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = sc[r] * c;
      if (!full_tile) {
        const int key = kb + 8 * (r >> 2) + 4 * grp + (r & 3);
        const bool ok = key < T && (!a.causal || key <= pos);
        v = ok ? v : -INFINITY;
      }
      sc[r] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    if (__any(mn > m)) {
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      m = mn;
    }
    // probabilities as bf16 pairs: slice t = registers 8t .. 8t+7
    uint32_t P[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P[t][i] = pack_bf16(fast_exp2(sc[8 * t + 2 * i] - m), fast_exp2(sc[8 * t + 2 * i + 1] - m));
        lsum = dot2_bf16(P[t][i], 0x3F803F80u, lsum);
      }
    // O^T += V^T P^T; k index (grp, e) of slice t <-> key 16t + 8(e/4) + 4 grp + e%4
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint8_t* vrow = lds_v + (32 * dt + lr) * LD::VROW;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint2 lo = *(const uint2*)(vrow + (16 * t + 4 * grp) * 2);
        const uint2 hi = *(const uint2*)(vrow + (16 * t + 8 + 4 * grp) * 2);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(P[t][0], P[t][1], P[t][2], P[t][3]));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // normalise and store: lane holds dims 32dt + 8(r/4) + 4grp + (0..3) of its row
  const float ltot = lsum + shfl_xor(lsum, 32);
  if (row_ok) {
    const float inv = ltot > 0.0f ? a.out_scale / ltot : 0.0f;
    uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + qi) * n_q + head) * HD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * grp;
        const uint32_t w0 = pack_bf16(acc[dt][4 * r4 + 0] * inv, acc[dt][4 * r4 + 1] * inv);
        const uint32_t w1 = pack_bf16(acc[dt][4 * r4 + 2] * inv, acc[dt][4 * r4 + 3] * inv);
        *(uint2*)(orow + d) = make_uint2(w0, w1);
      }
  }
}

template <int CDT, int HD>
static bool prefill_dispatch_g(int G, const PrefillArgs& a, unsigned grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<CDT, HD, 1>), dim3(grid), dim3(256), 0, st, a); return true;
    case 2: hipLaunchKernelGGL((prefill_kernel<CDT, HD, 2>), dim3(grid), dim3(256), 0, st, a); return true;
    case 4: hipLaunchKernelGGL((prefill_kernel<CDT, HD, 4>), dim3(grid), dim3(256), 0, st, a); return true;
    case 8: hipLaunchKernelGGL((prefill_kernel<CDT, HD, 8>), dim3(grid), dim3(256), 0, st, a); return true;
    default: return false;
  }
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t max_context_len) {
  (void)num_seqs; (void)total_q; (void)max_q_len; (void)n_q_heads; (void)n_kv_heads;
  (void)head_dim; (void)max_context_len;
  return 0;
}

extern "C" pa_status pa_prefill_chunk(void* out, const void* q, int q_dtype,
                                      const int32_t* cu_seqlens_q, int32_t num_seqs,
                                      int32_t total_q, int32_t max_q_len, const void* k_cache,
                                      const void* v_cache, int cache_dtype, int32_t num_blocks,
                                      int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t group_size, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t max_context_len, int32_t causal, float scale,
                                      float k_scale, float v_scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes; (void)max_context_len;
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || n_kv_heads < 1 ||
      max_blocks_per_seq < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1))) return PA_ERR_UNSUPPORTED;
  if (group_size != 1 && group_size != 2 && group_size != 4 && group_size != 8)
    return PA_ERR_UNSUPPORTED;
  if (q_dtype != PA_BF16 || (cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3))
    return PA_ERR_DTYPE;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !cu_seqlens_q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f))) return PA_ERR_SHAPE;
  PrefillArgs a;
  a.q = (const uint8_t*)q;
  a.out = out;
  a.cu_q = cu_seqlens_q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.tok_stride = (int64_t)n_kv_heads * head_dim * (fp8 ? 1 : 2);
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  a.bs_log2 = lg;
  a.n_kv = n_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  const int QB = PF_ROWS / group_size;
  a.qtiles = (max_q_len + QB - 1) / QB;
  a.causal = causal != 0;
  a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 ? v_scale : 1.0f;
  const int64_t grid = (int64_t)num_seqs * a.qtiles * n_kv_heads;
  if (grid >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  bool ok;
  if (cache_dtype == PA_BF16)
    ok = head_dim == 128 ? prefill_dispatch_g<PA_BF16, 128>(group_size, a, (unsigned)grid, st)
                         : prefill_dispatch_g<PA_BF16, 64>(group_size, a, (unsigned)grid, st);
  else
    ok = head_dim == 128 ? prefill_dispatch_g<PA_FP8_E4M3, 128>(group_size, a, (unsigned)grid, st)
                         : prefill_dispatch_g<PA_FP8_E4M3, 64>(group_size, a, (unsigned)grid, st);
  if (!ok) return PA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Paged decode attention: split kernel + log-sum-exp merge kernel.
//
// What is computed (the pages' definitions):
//   * attention of the step's query over K_{1:t}, V_{1:t} -- "KV Cache: the
//     memory bottleneck of LLM inference" (tag-page excerpt), section 1.1;
//   * K/V gathered through the block table, token p in block
//     table[p / block_size] at offset p % block_size -- "3.3 Batching and
//     memory management", section "PagedAttention: the block table";
//   * softmax accumulated block by block with the online recurrence
//     m_i = max(m_{i-1}, rowmax S_i), l_i = e^{m_{i-1}-m_i} l_{i-1} + rowsum e^{S_i-m_i},
//     O_i = e^{m_{i-1}-m_i} O_{i-1} + e^{S_i-m_i} V_i, divided by l at the end --
//     "From PagedAttention to Chunked Prefill", section 2.2 (the printed inverse
//     on the O rescale factor is read as belonging to the final division);
//   * split partials (m, l, O) combined by the same recurrence applied to whole
//     splits (the log-sum-exp merge).
//
// How it maps to CDNA4 (gfx950, wave64):
//   * One wave = one (sequence, KV head, split).  It owns all group_size query
//     heads of that KV head, so every K/V byte is fetched from HBM exactly once.
//   * Lane l works on token slot g = l >> 3 (and g + 8) of each 16-token step and
//     on the dims of lane column c = l & 7.  One 16-byte load per lane covers 8
//     tokens x 128 contiguous bytes: whole cache lines, fully coalesced, with no
//     LDS round trip (each byte is used by exactly one lane).
//   * Scores: v_dot2_f32_bf16 over bf16 pairs (fp8 codes are widened to bf16
//     pairs exactly with the gfx950 pair converter), then a 3-step DPP sum over
//     the 8 lanes of the token.
//   * Softmax is lane-local: each group of 8 lanes keeps its own running max,
//     sum and accumulator over the tokens it has seen, so a step needs no
//     cross-lane max; the rescale of the accumulator runs only when some lane's
//     max grew (a wave-uniform branch, rare after the first steps).  The 8
//     groups are merged once at the end of the split.
//   * PV: the two token slots of a lane form the bf16 pair of v_dot2, so the
//     probabilities are packed once per step with v_cvt_pk_bf16_f32 and the sum
//     l is accumulated from the same rounded weights.  fp32 caches take an fp32
//     FMA path instead (no rounding of the weights).
//   * K/V of the next step are in flight while the current one is computed.
#include "pa_device.h"

namespace pa {

template <int CDT, int HD>
struct DecodeLayout {
  static constexpr int EB = CDT == PA_F32 ? 4 : CDT == PA_BF16 ? 2 : 1;
  static constexpr int ROW = HD * EB;                   // bytes of one (token, head) row
  static constexpr int LANE = ROW / 8;                  // bytes per lane per token
  static constexpr int CHUNK = LANE >= 16 ? 16 : LANE;  // bytes per load instruction
  static constexpr int NCHUNK = LANE / CHUNK;
  static constexpr int DW = LANE / 4;                   // dwords per lane per token
  static constexpr int DPL = HD / 8;                    // dims per lane
  static constexpr int EPC = CHUNK / EB;                // elements per chunk
  static constexpr bool F32 = CDT == PA_F32;
  static constexpr int QDW = F32 ? DPL : DPL / 2;       // q dwords per head per lane
};

struct DecodeArgs {
  const uint8_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;      // [num_seqs][n_q][max_splits][HD]
  float* part_ml;     // [num_seqs][n_q][max_splits][2]
  int64_t tok_stride; // bytes between consecutive tokens of a block (n_kv * ROW)
  int num_blocks;
  int block_size;
  int bs_log2;
  int n_kv;
  int max_blocks;
  int max_splits;
  int min_split;
  float score_scale;  // scale * k_scale * log2(e)
};

template <class L>
struct Frag {
  uint32_t k[2][L::DW];
  uint32_t v[2][L::DW];
  bool ok[2];
};

template <class L>
__device__ __forceinline__ void load_row(const uint8_t* p, uint32_t (&d)[L::DW]) {
#pragma unroll
  for (int k = 0; k < L::NCHUNK; ++k) {
    if constexpr (L::CHUNK == 16) {
      const uint4 x = *(const uint4*)(p + k * 8 * L::CHUNK);
      d[4 * k + 0] = x.x; d[4 * k + 1] = x.y; d[4 * k + 2] = x.z; d[4 * k + 3] = x.w;
    } else {
      const uint2 x = *(const uint2*)(p + k * 8 * L::CHUNK);
      d[2 * k + 0] = x.x; d[2 * k + 1] = x.y;
    }
  }
}

template <class L>
__device__ __forceinline__ void zero_frag(Frag<L>& f) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < L::DW; ++i) { f.k[j][i] = 0u; f.v[j][i] = 0u; }
}

// Issue the loads of one 16-token step starting at token `base` (a multiple of 16).
// Token slots whose position is >= end, or whose block id is outside the pool,
// are not loaded: their registers are zero and ok[] is false.
template <class L>
__device__ __forceinline__ void load_step(Frag<L>& f, const DecodeArgs& a, const int32_t* table,
                                          int base, int end, int kvh, int lane_g,
                                          int lane_byte) {
  const bool full = base + 16 <= end;
  const int64_t head_off = (int64_t)kvh * L::ROW + lane_byte;
  if (a.block_size >= 16) {
    // all 16 tokens of the step sit in one block: one (scalar) table read
    const int j = base >> a.bs_log2;
    const int blk = j < a.max_blocks ? table[j] : -1;
    const bool blk_ok = (unsigned)blk < (unsigned)a.num_blocks;
    const int64_t o0 = ((int64_t)blk * a.block_size + (base & (a.block_size - 1)) + lane_g) *
                           a.tok_stride + head_off;
    if (full && blk_ok) {           // wave-uniform fast path
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f.ok[j] = true;
        load_row<L>(a.k_cache + o0 + 8 * j * a.tok_stride, f.k[j]);
        load_row<L>(a.v_cache + o0 + 8 * j * a.tok_stride, f.v[j]);
      }
      return;
    }
    zero_frag<L>(f);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = blk_ok && base + lane_g + 8 * j < end;
      f.ok[j] = ok;
      if (ok) {
        load_row<L>(a.k_cache + o0 + 8 * j * a.tok_stride, f.k[j]);
        load_row<L>(a.v_cache + o0 + 8 * j * a.tok_stride, f.v[j]);
      }
    }
  } else {
    zero_frag<L>(f);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = base + lane_g + 8 * j;
      bool ok = pos < end;
      int blk = 0;
      if (ok) {
        const int jb = pos >> a.bs_log2;
        blk = jb < a.max_blocks ? table[jb] : -1;
        ok = (unsigned)blk < (unsigned)a.num_blocks;
      }
      f.ok[j] = ok;
      if (ok) {
        const int64_t o = ((int64_t)blk * a.block_size + (pos & (a.block_size - 1))) * a.tok_stride + head_off;
        load_row<L>(a.k_cache + o, f.k[j]);
        load_row<L>(a.v_cache + o, f.v[j]);
      }
    }
  }
}

template <int CDT, int HD, int G>
struct DecodeState {
  using L = DecodeLayout<CDT, HD>;
  uint32_t q[G][L::QDW];
  float o[G][L::DPL];
  float m[G];
  float l[G];
};

// Score of one token for every head of the group (partial over this lane's dims).
template <int CDT, int HD, int G>
__device__ __forceinline__ void lane_scores(const DecodeState<CDT, HD, G>& st,
                                            const uint32_t (&kd)[DecodeLayout<CDT, HD>::DW],
                                            float (&s)[G]) {
  using L = DecodeLayout<CDT, HD>;
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.0f;
  if constexpr (CDT == PA_BF16) {
#pragma unroll
    for (int i = 0; i < L::DW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = dot2_bf16(st.q[h][i], kd[i], s[h]);
  } else if constexpr (CDT == PA_FP8_E4M3) {
#pragma unroll
    for (int i = 0; i < L::DW; ++i) {
      const uint32_t lo = fp8x2_to_bf16x2<false>(kd[i]);
      const uint32_t hi = fp8x2_to_bf16x2<true>(kd[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = dot2_bf16(st.q[h][2 * i], lo, s[h]);
        s[h] = dot2_bf16(st.q[h][2 * i + 1], hi, s[h]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < L::DW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = fmaf(bits_f32(st.q[h][i]), bits_f32(kd[i]), s[h]);
  }
}

template <int CDT, int HD, int G>
__device__ __forceinline__ void process_step(DecodeState<CDT, HD, G>& st,
                                             const Frag<DecodeLayout<CDT, HD>>& f, float c) {
  using L = DecodeLayout<CDT, HD>;
  float s0[G], s1[G];
  lane_scores<CDT, HD, G>(st, f.k[0], s0);
  lane_scores<CDT, HD, G>(st, f.k[1], s1);
  bool grow = false;
  float mn[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float t0 = sum8(s0[h]) * c;   // all 8 lanes of a token share ok[]
    const float t1 = sum8(s1[h]) * c;
    s0[h] = f.ok[0] ? t0 : -INFINITY;
    s1[h] = f.ok[1] ? t1 : -INFINITY;
    mn[h] = fmaxf(st.m[h], fmaxf(s0[h], s1[h]));
    grow |= mn[h] > st.m[h];
  }
  if (__any(grow)) {   // wave-uniform: rescale to the new running max
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = fast_exp2(st.m[h] - mn[h]);
      st.m[h] = mn[h];
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < L::DPL; ++e) st.o[h][e] *= alpha;
    }
  }
  if constexpr (L::F32) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p0 = fast_exp2(s0[h] - st.m[h]);
      const float p1 = fast_exp2(s1[h] - st.m[h]);
      st.l[h] += p0 + p1;
#pragma unroll
      for (int e = 0; e < L::DPL; ++e)
        st.o[h][e] = fmaf(p0, bits_f32(f.v[0][e]), fmaf(p1, bits_f32(f.v[1][e]), st.o[h][e]));
    }
  } else {
    uint32_t P[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      P[h] = pack_bf16(fast_exp2(s0[h] - st.m[h]), fast_exp2(s1[h] - st.m[h]));
      st.l[h] = dot2_bf16(P[h], 0x3F803F80u, st.l[h]);   // sum of the rounded weights
    }
    if constexpr (CDT == PA_BF16) {
#pragma unroll
      for (int i = 0; i < L::DW; ++i) {
        const uint32_t lo = pair_lo(f.v[0][i], f.v[1][i]);   // dim 2i of both tokens
        const uint32_t hi = pair_hi(f.v[0][i], f.v[1][i]);   // dim 2i+1
#pragma unroll
        for (int h = 0; h < G; ++h) {
          st.o[h][2 * i] = dot2_bf16(P[h], lo, st.o[h][2 * i]);
          st.o[h][2 * i + 1] = dot2_bf16(P[h], hi, st.o[h][2 * i + 1]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < L::DW; ++i) {
        const uint32_t a0 = fp8x2_to_bf16x2<false>(f.v[0][i]);
        const uint32_t b0 = fp8x2_to_bf16x2<false>(f.v[1][i]);
        const uint32_t a1 = fp8x2_to_bf16x2<true>(f.v[0][i]);
        const uint32_t b1 = fp8x2_to_bf16x2<true>(f.v[1][i]);
        const uint32_t d0 = pair_lo(a0, b0), d1 = pair_hi(a0, b0);
        const uint32_t d2 = pair_lo(a1, b1), d3 = pair_hi(a1, b1);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          st.o[h][4 * i + 0] = dot2_bf16(P[h], d0, st.o[h][4 * i + 0]);
          st.o[h][4 * i + 1] = dot2_bf16(P[h], d1, st.o[h][4 * i + 1]);
          st.o[h][4 * i + 2] = dot2_bf16(P[h], d2, st.o[h][4 * i + 2]);
          st.o[h][4 * i + 3] = dot2_bf16(P[h], d3, st.o[h][4 * i + 3]);
        }
      }
    }
  }
}

// Dim index of element e of a lane's fragment (lane column c).
template <class L>
__device__ __forceinline__ int lane_dim(int c, int e) {
  const int k = e / L::EPC, w = e % L::EPC;
  return (k * 8 * L::CHUNK + c * L::CHUNK) / L::EB + w;
}

template <int CDT, int HD, int G>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using L = DecodeLayout<CDT, HD>;
  const int lane = threadIdx.x;
  const int lane_g = lane >> 3, lane_c = lane & 7;
  int wid = blockIdx.x;
  const int split = wid % a.max_splits;
  wid /= a.max_splits;
  const int kvh = wid % a.n_kv;
  const int s = wid / a.n_kv;
  const int ctx = a.context_lens[s];
  int ns, slen;
  decode_plan(ctx, a.max_splits, a.min_split, &ns, &slen);
  if (split >= ns) return;
  const int begin = split * slen;
  const int end = min(ctx, begin + slen);
  const int n_q = a.n_kv * G;

  DecodeState<CDT, HD, G> st;
  // query fragment: the same dims as this lane's K/V elements
  {
    constexpr int QEB = L::F32 ? 4 : 2;
    const uint8_t* qrow = a.q + ((int64_t)s * n_q + (int64_t)kvh * G) * HD * QEB;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int k = 0; k < L::NCHUNK; ++k) {
        const int d0 = lane_dim<L>(lane_c, k * L::EPC);
        const uint8_t* p = qrow + ((int64_t)h * HD + d0) * QEB;
        constexpr int QD = L::EPC * QEB / 4;     // q dwords for one chunk
#pragma unroll
        for (int i = 0; i < QD; i += 4) {
          const uint4 x = *(const uint4*)(p + 4 * i);
          st.q[h][k * QD + i + 0] = x.x; st.q[h][k * QD + i + 1] = x.y;
          st.q[h][k * QD + i + 2] = x.z; st.q[h][k * QD + i + 3] = x.w;
        }
      }
      st.m[h] = -1e30f;
      st.l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < L::DPL; ++e) st.o[h][e] = 0.0f;
    }
  }

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const int lane_byte = lane_c * L::CHUNK;
  const float c = a.score_scale;

  // two fragments in flight: compute one step while the next one loads
  Frag<L> fa, fb;
  int base = begin;
  load_step<L>(fa, a, table, base, end, kvh, lane_g, lane_byte);
  while (true) {
    const int nb = base + 16;
    if (nb < end) load_step<L>(fb, a, table, nb, end, kvh, lane_g, lane_byte);
    process_step<CDT, HD, G>(st, fa, c);
    if (nb >= end) break;
    const int nn = nb + 16;
    if (nn < end) load_step<L>(fa, a, table, nn, end, kvh, lane_g, lane_byte);
    process_step<CDT, HD, G>(st, fb, c);
    if (nn >= end) break;
    base = nn;
  }

  // merge the 8 lane groups (lane-local softmax states) of this wave
  float* out_o = a.part_o + (((int64_t)s * n_q + (int64_t)kvh * G) * a.max_splits + split) * HD;
  float* out_ml = a.part_ml + (((int64_t)s * n_q + (int64_t)kvh * G) * a.max_splits + split) * 2;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = max_over_groups(st.m[h]);
    const float w = fast_exp2(st.m[h] - M);
    const float lsum = sum_over_groups(st.l[h] * w);
    float ov[L::DPL];
#pragma unroll
    for (int e = 0; e < L::DPL; ++e) ov[e] = sum_over_groups(st.o[h][e] * w);
    if (lane_g == h) {   // lanes of group h store head h
      float* dst = out_o + (int64_t)h * a.max_splits * HD;
#pragma unroll
      for (int k = 0; k < L::NCHUNK; ++k) {
        const int d0 = lane_dim<L>(lane_c, k * L::EPC);
#pragma unroll
        for (int i = 0; i < L::EPC; i += 4)
          *(float4*)(dst + d0 + i) = make_float4(ov[k * L::EPC + i], ov[k * L::EPC + i + 1],
                                                 ov[k * L::EPC + i + 2], ov[k * L::EPC + i + 3]);
      }
      if (lane_c == 0)
        *(float2*)(out_ml + (int64_t)h * a.max_splits * 2) = make_float2(M, lsum);
    }
  }
}

// One wave per (sequence, query head): combine the splits' (m, l, O).
template <int HD, bool OUT_BF16>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    void* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ context_lens, int n_q, int max_splits, int min_split,
    float v_scale) {
  constexpr int DPT = HD / 64;   // dims per thread
  const int h = blockIdx.x % n_q;
  const int s = blockIdx.x / n_q;
  const int t = threadIdx.x;
  int ns, slen;
  decode_plan(context_lens[s], max_splits, min_split, &ns, &slen);
  const int64_t row = (int64_t)s * n_q + h;
  const float* po = part_o + row * max_splits * HD;
  const float* pml = part_ml + row * max_splits * 2;
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.0f;
  float inv = 0.0f;
  if (ns > 0) {
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, pml[2 * k]);
    float lsum = 0.0f;
    for (int k = 0; k < ns; ++k) {
      const float w = fast_exp2(pml[2 * k] - M);
      lsum = fmaf(w, pml[2 * k + 1], lsum);
#pragma unroll
      for (int i = 0; i < DPT; ++i) acc[i] = fmaf(w, po[(int64_t)k * HD + t * DPT + i], acc[i]);
    }
    inv = v_scale / lsum;
  }
  if constexpr (OUT_BF16) {
    uint16_t* o = (uint16_t*)out + row * HD + t * DPT;
    if constexpr (DPT == 2) {
      *(uint32_t*)o = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      o[0] = (uint16_t)(pack_bf16(acc[0] * inv, 0.0f) & 0xffffu);
    }
  } else {
    float* o = (float*)out + row * HD + t * DPT;
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[i] = acc[i] * inv;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct HostPlan {
  int max_splits;
  int min_split;
};

static HostPlan host_plan(int max_context_len, int split_tokens) {
  HostPlan p;
  const int ctx = max_context_len > 0 ? max_context_len : 1;
  if (split_tokens > 0) {
    p.min_split = (split_tokens + 15) & ~15;
    p.max_splits = (ctx + p.min_split - 1) / p.min_split;
  } else {
    p.min_split = 256;
    p.max_splits = (ctx + p.min_split - 1) / p.min_split;
    if (p.max_splits > 64) p.max_splits = 64;
  }
  if (p.max_splits < 1) p.max_splits = 1;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t workspace_for(int num_seqs, int n_q, int head_dim, const HostPlan& p) {
  const size_t rows = (size_t)num_seqs * n_q * p.max_splits;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

template <int CDT, int HD, int G>
static void launch_split(const DecodeArgs& a, int num_seqs, hipStream_t st) {
  const unsigned grid = (unsigned)((int64_t)a.max_splits * a.n_kv * num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<CDT, HD, G>), dim3(grid), dim3(64), 0, st, a);
}

template <int CDT, int HD>
static bool dispatch_group(int G, const DecodeArgs& a, int num_seqs, hipStream_t st) {
  switch (G) {
    case 1: launch_split<CDT, HD, 1>(a, num_seqs, st); return true;
    case 2: launch_split<CDT, HD, 2>(a, num_seqs, st); return true;
    case 4: launch_split<CDT, HD, 4>(a, num_seqs, st); return true;
    case 8: launch_split<CDT, HD, 8>(a, num_seqs, st); return true;
    default: return false;
  }
}

template <int CDT>
static bool dispatch_hd(int hd, int G, const DecodeArgs& a, int num_seqs, hipStream_t st) {
  if (hd == 128) return dispatch_group<CDT, 128>(G, a, num_seqs, st);
  if (hd == 64) return dispatch_group<CDT, 64>(G, a, num_seqs, st);
  return false;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                            int32_t n_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t split_tokens) {
  (void)n_kv_heads;
  if (num_seqs <= 0 || n_q_heads <= 0 || head_dim <= 0) return 0;
  return workspace_for(num_seqs, n_q_heads, head_dim, host_plan(max_context_len, split_tokens));
}

extern "C" pa_status pa_decode(void* out, const void* q, int q_dtype, const void* k_cache,
                               const void* v_cache, int cache_dtype, int32_t num_blocks,
                               int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                               int32_t group_size, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t max_context_len, float scale,
                               float k_scale, float v_scale, int32_t split_tokens,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_blocks < 0 || n_kv_heads < 1 || group_size < 1 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || split_tokens < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1))) return PA_ERR_UNSUPPORTED;
  if (group_size != 1 && group_size != 2 && group_size != 4 && group_size != 8)
    return PA_ERR_UNSUPPORTED;
  const bool pair_ok = (q_dtype == PA_F32 && cache_dtype == PA_F32) ||
                       (q_dtype == PA_BF16 && (cache_dtype == PA_BF16 || cache_dtype == PA_FP8_E4M3));
  if (!pair_ok) return PA_ERR_DTYPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  const int n_q = n_kv_heads * group_size;
  const HostPlan plan = host_plan(max_context_len, split_tokens);
  const size_t need = workspace_for(num_seqs, n_q, head_dim, plan);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return PA_ERR_WORKSPACE;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f))) return PA_ERR_SHAPE;

  DecodeArgs a;
  a.q = (const uint8_t*)q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t rows = (size_t)num_seqs * n_q * plan.max_splits;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + align256(rows * head_dim * sizeof(float)));
  const int eb = cache_dtype == PA_F32 ? 4 : cache_dtype == PA_BF16 ? 2 : 1;
  a.tok_stride = (int64_t)n_kv_heads * head_dim * eb;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  a.bs_log2 = lg;
  a.n_kv = n_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_splits = plan.max_splits;
  a.min_split = plan.min_split;
  a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;

  hipStream_t st = (hipStream_t)stream;
  bool ok = false;
  if (cache_dtype == PA_BF16) ok = dispatch_hd<PA_BF16>(head_dim, group_size, a, num_seqs, st);
  else if (cache_dtype == PA_FP8_E4M3) ok = dispatch_hd<PA_FP8_E4M3>(head_dim, group_size, a, num_seqs, st);
  else ok = dispatch_hd<PA_F32>(head_dim, group_size, a, num_seqs, st);
  if (!ok) return PA_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;

  const unsigned mgrid = (unsigned)((int64_t)num_seqs * n_q);
  const float vs = fp8 ? v_scale : 1.0f;
  if (q_dtype == PA_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<128, true>), dim3(mgrid), dim3(64), 0, st, out,
                         a.part_o, a.part_ml, context_lens, n_q, plan.max_splits, plan.min_split, vs);
    else
      hipLaunchKernelGGL((decode_merge_kernel<64, true>), dim3(mgrid), dim3(64), 0, st, out,
                         a.part_o, a.part_ml, context_lens, n_q, plan.max_splits, plan.min_split, vs);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<128, false>), dim3(mgrid), dim3(64), 0, st, out,
                         a.part_o, a.part_ml, context_lens, n_q, plan.max_splits, plan.min_split, vs);
    else
      hipLaunchKernelGGL((decode_merge_kernel<64, false>), dim3(mgrid), dim3(64), 0, st, out,
                         a.part_o, a.part_ml, context_lens, n_q, plan.max_splits, plan.min_split, vs);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

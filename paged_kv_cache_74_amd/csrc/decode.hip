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
// Two split kernels share the work split, the partial format and the merge:
//   * decode_mfma_kernel (further below): both products on the matrix cores;
//     taken for bf16, fp8, int8 and int4 caches with blocks of >= 16 tokens;
//   * decode_split_kernel (this part): the products on the vector ALU; taken
//     for fp32 caches and for blocks of fewer than 16 tokens.
//
// How the vector kernel maps to CDNA4 (gfx950, wave64):
//   * One wave = one (sequence, KV head, split).  It owns all group_size query
//     heads of that KV head, so every K/V byte is fetched from HBM exactly once.
//     The waves of a workgroup take consecutive KV heads of the same sequence
//     and steps: together they read whole token rows of each block (all heads
//     of a token are adjacent in the pool), so HBM sees long contiguous runs
//     instead of one 256-byte row per token.
//   * Lane l works on token slot g = l >> 3 (and g + 8) of each 16-token step and
//     on the dims of lane column c = l & 7.  One 16-byte load per lane covers 8
//     tokens x 128 contiguous bytes: whole cache lines, fully coalesced, with no
//     LDS round trip (each byte is used by exactly one lane).
//   * Scores: v_dot2_f32_bf16 over bf16 pairs (fp8 and int8 codes are widened to bf16
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
#include "internal.h"

#include <mutex>

namespace pa {

template <int CDT, int HD>
struct DecodeLayout {
  static constexpr int EBITS = CDT == PA_F32 ? 32 : CDT == PA_BF16 ? 16 : CDT == PA_INT4 ? 4 : 8;
  static constexpr int ROW = HD * EBITS / 8;            // bytes of one (token, head) row
  static constexpr int LANE = ROW / 8;                  // bytes per lane per token
  static constexpr int CHUNK = LANE >= 16 ? 16 : LANE;  // bytes per load instruction
  static constexpr int NCHUNK = LANE / CHUNK;
  static constexpr int DW = LANE / 4;                   // dwords per lane per token
  static constexpr int DPL = HD / 8;                    // dims per lane
  static constexpr int EPC = CHUNK * 8 / EBITS;         // elements per chunk
  static constexpr bool F32 = CDT == PA_F32;
  static constexpr int QDW = F32 ? DPL : DPL / 2;       // q dwords per head per lane
};

#ifndef DECODE_LOAD_AUX
#define DECODE_LOAD_AUX 2   // K/V loads are streamed once: non-temporal ("nt") cache policy
#endif
#ifndef DECODE_NBUF
#define DECODE_NBUF 2   // K/V steps resident per wave: NBUF - 1 in flight during compute
#endif
#ifndef DECODE_MAX_HW
#define DECODE_MAX_HW 8   // most KV heads (waves) per workgroup
#endif
// With 8 query heads per KV head (4 for fp32 caches) a wave needs more than 256
// registers: at most 4 waves per workgroup then, so that a workgroup fits the
// register file.
__host__ __device__ constexpr int max_hw(int CDT, int G) {
  return (G >= 8 || (CDT == PA_F32 && G >= 4)) ? 4 : DECODE_MAX_HW;
}
#ifndef DECODE_WAVES_PER_CU
#define DECODE_WAVES_PER_CU 16   // resident waves per CU the split kernel is launched with
#endif

struct DecodeArgs {
  const uint8_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* header;           // {workgroups, waves per workgroup, start-up units, units}, for the merge
  int32_t* seg_w;            // [segments][2]: workgroups that ran a segment's first and last step
  float* part_o;      // [slots][HW][G][HD]   slot = workgroup + segment
  float* part_ml;     // [slots][HW][G][2]
  int64_t tok_stride; // bytes between consecutive tokens of a block (n_kv * ROW)
  int num_blocks;
  int block_size;
  int bs_log2;
  int n_kv;
  int max_blocks;
  int num_seqs;
  int num_wgs;
  int hw;             // waves (KV heads) per workgroup; n_kv = hw * nhg
  int nhg;            // KV head groups
  float score_scale;  // scale * k_scale * log2(e)
  const float* k_ch_scale;   // INT4: [n_kv][HD] key scale per channel
  const float* v_tok_scale;  // INT4: [num_blocks][n_kv][block_size] value scale per token
  // vector kernel only: block-table row of each query row (NULL: row s reads
  // table row s).  The fp32 chunked prefill runs each query row as a decode
  // row of its own sequence.
  const int32_t* table_row;
  // matrix-core kernel and merge: the q and out row of sequence s (a query row
  // of a ragged batch; -1: the sequence has no row here), NULL: row s.  The
  // chunked prefill runs its query-length-1 rows through this path.
  const int32_t* row_map;
  // The appending decode: token context_lens[s] - 1 of every sequence is
  // k_new[s] / v_new[s] ([num_seqs][n_kv][HD] of the source dtype), written to
  // its slot (as pa_kv_append writes it) by the workgroup that reads it
  const uint8_t* k_new;
  const uint8_t* v_new;
  int src_f32;               // source dtype: F32 (1) or BF16 (0)
  float k_inv, v_inv;        // 8-bit caches: 1 / scale, binary32
  int64_t* slots_out;        // optional: the appended tokens' slots
};

// 16 cache bytes of a new token row from its source elements, starting at
// source element e0: a bit copy (F32 or BF16 cache from the same dtype) or 16
// codes encoded as pa_kv_append encodes them (FP8_E4M3 or INT8 cache).
template <int CDT>
__device__ __forceinline__ uint4 new_chunk(const uint8_t* src, int64_t e0, bool src_f32, float inv) {
  if constexpr (CDT == PA_F32) {
    return *(const uint4*)(src + e0 * 4);
  } else if constexpr (CDT == PA_BF16) {
    return *(const uint4*)(src + e0 * 2);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (src_f32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 x = *(const uint4*)(src + (e0 + 4 * q) * 4);
        const uint32_t v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) w[q] |= encode8<CDT>(bits_f32(v[e]) * inv) << (8 * e);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 x = *(const uint4*)(src + (e0 + 8 * q) * 2);
        const uint32_t v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = encode8<CDT>(bf16lo_f32(v[e]) * inv);
          const uint32_t hi = encode8<CDT>(bf16hi_f32(v[e]) * inv);
          w[2 * q + (e >> 1)] |= (lo | (hi << 8)) << (16 * (e & 1));
        }
      }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Slot of token p of a sequence through its table row, or -1 (a negative
// entry, or p past the row).
__device__ __forceinline__ int64_t row_slot(const int32_t* row, int max_blocks, int block_size,
                                            int bs_log2, int p) {
  if (p < 0 || (p >> bs_log2) >= max_blocks) return -1;
  const int32_t blk = row[p >> bs_log2];
  return blk >= 0 ? (int64_t)blk * block_size + (p & (block_size - 1)) : -1;
}

template <class L>
struct Frag {
  uint32_t k[2][L::DW];
  uint32_t v[2][L::DW];
  float vs[2];   // INT4: the value scales of the two token slots
  bool ok[2];
};

template <class L>
__device__ __forceinline__ void load_row(const uint8_t* p, uint32_t (&d)[L::DW]) {
#pragma unroll
  for (int k = 0; k < L::NCHUNK; ++k) {
    if constexpr (L::CHUNK == 16) {
      const uint4 x = *(const uint4*)(p + k * 8 * L::CHUNK);
      d[4 * k + 0] = x.x; d[4 * k + 1] = x.y; d[4 * k + 2] = x.z; d[4 * k + 3] = x.w;
    } else if constexpr (L::CHUNK == 8) {
      const uint2 x = *(const uint2*)(p + k * 8 * L::CHUNK);
      d[2 * k + 0] = x.x; d[2 * k + 1] = x.y;
    } else {
      d[k] = *(const uint32_t*)(p + k * 8 * L::CHUNK);
    }
  }
}

// Buffer loads: a wave-uniform descriptor (base address in scalar registers)
// plus a per-lane 32-bit byte offset, so no 64-bit per-lane address is built.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  // 4th descriptor word for the gfx9 family: 32-bit data format, raw addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <class L>
__device__ __forceinline__ void load_row_b(__amdgpu_buffer_rsrc_t r, uint32_t voff, int32_t soff,
                                           uint32_t (&d)[L::DW]) {
#pragma unroll
  for (int k = 0; k < L::NCHUNK; ++k) {
    if constexpr (L::CHUNK == 16) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff + k * 8 * L::CHUNK, soff, DECODE_LOAD_AUX);
      d[4 * k + 0] = x.x; d[4 * k + 1] = x.y; d[4 * k + 2] = x.z; d[4 * k + 3] = x.w;
    } else if constexpr (L::CHUNK == 8) {
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff + k * 8 * L::CHUNK, soff, DECODE_LOAD_AUX);
      d[2 * k + 0] = x.x; d[2 * k + 1] = x.y;
    } else {
      d[k] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + k * 8 * L::CHUNK, soff, DECODE_LOAD_AUX);
    }
  }
}

template <class L>
__device__ __forceinline__ void zero_frag(Frag<L>& f) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < L::DW; ++i) { f.k[j][i] = 0u; f.v[j][i] = 0u; }
    f.vs[j] = 0.0f;
  }
}

// INT4: the value scale of token `tok` (its index in the pool) for KV head kvh.
template <class L>
__device__ __forceinline__ float token_scale(const DecodeArgs& a, int64_t tok, int kvh) {
  if constexpr (L::EBITS == 4)
    return a.v_tok_scale[((tok >> a.bs_log2) * a.n_kv + kvh) * a.block_size +
                         (tok & (a.block_size - 1))];
  else return 0.0f;
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
    const int blk = j < a.max_blocks ? uniform_load(table, j) : -1;
    const bool blk_ok = (unsigned)blk < (unsigned)a.num_blocks;
    const int64_t t0 = (int64_t)blk * a.block_size + (base & (a.block_size - 1)) + lane_g;
    const int64_t o0 = t0 * a.tok_stride + head_off;
    if (full && blk_ok) {           // wave-uniform fast path
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f.ok[j] = true;
        load_row<L>(a.k_cache + o0 + 8 * j * a.tok_stride, f.k[j]);
        load_row<L>(a.v_cache + o0 + 8 * j * a.tok_stride, f.v[j]);
        f.vs[j] = token_scale<L>(a, t0 + 8 * j, kvh);
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
        f.vs[j] = token_scale<L>(a, t0 + 8 * j, kvh);
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
        const int64_t t = (int64_t)blk * a.block_size + (pos & (a.block_size - 1));
        const int64_t o = t * a.tok_stride + head_off;
        load_row<L>(a.k_cache + o, f.k[j]);
        load_row<L>(a.v_cache + o, f.v[j]);
        f.vs[j] = token_scale<L>(a, t, kvh);
      }
    }
  }
}

// Loads of one full 16-token step when block_size >= 16 (the step lies in one
// block).  The same 4 * NCHUNK loads are issued on every path, so the number
// of loads in flight is fixed and the compiler's waits stay tight.  A block id
// outside the pool is never dereferenced (block 0 is read instead).
// With live == false the loads are still issued (keeping the count in flight
// fixed) but through an empty descriptor: they return zeros and touch no memory.
template <class L>
__device__ __forceinline__ void load_full_step(Frag<L>& f, const DecodeArgs& a,
                                               const int32_t* table, int base, uint32_t lane_off,
                                               bool live, int kvh, int lane_g) {
  const int j = base >> a.bs_log2;
  int blk = j < a.max_blocks ? uniform_load(table, j) : 0;
  blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
  const int64_t tok0 = (int64_t)blk * a.block_size + (base & (a.block_size - 1));
  const int64_t step_off = tok0 * a.tok_stride;
  if constexpr (L::EBITS == 4) {   // value scales of the lane's two token slots (in the pool)
    f.vs[0] = token_scale<L>(a, tok0 + lane_g, kvh);
    f.vs[1] = token_scale<L>(a, tok0 + lane_g + 8, kvh);
  }
  const int32_t step_bytes = live ? 16 * (int32_t)a.tok_stride : 0;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k_cache + step_off, step_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v_cache + step_off, step_bytes);
  const int32_t half = 8 * (int32_t)a.tok_stride;
  load_row_b<L>(kr, lane_off, 0, f.k[0]);
  load_row_b<L>(kr, lane_off, half, f.k[1]);
  load_row_b<L>(vr, lane_off, 0, f.v[0]);
  load_row_b<L>(vr, lane_off, half, f.v[1]);
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
  } else if constexpr (CDT == PA_FP8_E4M3 || CDT == PA_INT8) {
#pragma unroll
    for (int i = 0; i < L::DW; ++i) {
      const uint32_t lo = code8x2_to_bf16x2<CDT, false>(kd[i]);
      const uint32_t hi = code8x2_to_bf16x2<CDT, true>(kd[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = dot2_bf16(st.q[h][2 * i], lo, s[h]);
        s[h] = dot2_bf16(st.q[h][2 * i + 1], hi, s[h]);
      }
    }
  } else if constexpr (CDT == PA_INT4) {
    // dword i holds elements 8i .. 8i+7; the pairs come out as (0,2) (4,6)
    // (1,3) (5,7), the order the query pairs were packed in
#pragma unroll
    for (int i = 0; i < L::DW; ++i) {
      const uint32_t lo = int4_lo_as_e4m3(kd[i]), hi = int4_hi_as_e4m3(kd[i]);
      const uint32_t k0 = int4e4m3_to_bf16x2<false>(lo), k1 = int4e4m3_to_bf16x2<true>(lo);
      const uint32_t k2 = int4e4m3_to_bf16x2<false>(hi), k3 = int4e4m3_to_bf16x2<true>(hi);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = dot2_bf16(st.q[h][4 * i + 0], k0, s[h]);
        s[h] = dot2_bf16(st.q[h][4 * i + 1], k1, s[h]);
        s[h] = dot2_bf16(st.q[h][4 * i + 2], k2, s[h]);
        s[h] = dot2_bf16(st.q[h][4 * i + 3], k3, s[h]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < L::DW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = fmaf(bits_f32(st.q[h][i]), bits_f32(kd[i]), s[h]);
  }
}

template <int CDT, int HD, int G, bool MASKED>
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
    s0[h] = (!MASKED || f.ok[0]) ? t0 : -INFINITY;
    s1[h] = (!MASKED || f.ok[1]) ? t1 : -INFINITY;
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
  } else if constexpr (CDT == PA_INT4) {
    // A value is code * (its token's scale): the scale multiplies the weight
    // before it is rounded to bf16; l sums the unscaled weights in fp32.
    uint32_t P[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p0 = fast_exp2(s0[h] - st.m[h]), p1 = fast_exp2(s1[h] - st.m[h]);
      P[h] = pack_bf16(p0 * f.vs[0], p1 * f.vs[1]);
      st.l[h] += p0 + p1;
    }
#pragma unroll
    for (int i = 0; i < L::DW; ++i) {
      const uint32_t L0 = int4_lo_as_e4m3(f.v[0][i]), L1 = int4_lo_as_e4m3(f.v[1][i]);
      const uint32_t H0 = int4_hi_as_e4m3(f.v[0][i]), H1 = int4_hi_as_e4m3(f.v[1][i]);
      // bytes {t0, t1} of one element side by side: elements (0, 2), (4, 6), (1, 3), (5, 7)
      const uint32_t x0 = perm_b32(L1, L0, 0x05010400u), x1 = perm_b32(L1, L0, 0x07030602u);
      const uint32_t y0 = perm_b32(H1, H0, 0x05010400u), y1 = perm_b32(H1, H0, 0x07030602u);
      const uint32_t d0 = int4e4m3_to_bf16x2<false>(x0), d2 = int4e4m3_to_bf16x2<true>(x0);
      const uint32_t d4 = int4e4m3_to_bf16x2<false>(x1), d6 = int4e4m3_to_bf16x2<true>(x1);
      const uint32_t d1 = int4e4m3_to_bf16x2<false>(y0), d3 = int4e4m3_to_bf16x2<true>(y0);
      const uint32_t d5 = int4e4m3_to_bf16x2<false>(y1), d7 = int4e4m3_to_bf16x2<true>(y1);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* o = st.o[h] + 8 * i;
        o[0] = dot2_bf16(P[h], d0, o[0]); o[1] = dot2_bf16(P[h], d1, o[1]);
        o[2] = dot2_bf16(P[h], d2, o[2]); o[3] = dot2_bf16(P[h], d3, o[3]);
        o[4] = dot2_bf16(P[h], d4, o[4]); o[5] = dot2_bf16(P[h], d5, o[5]);
        o[6] = dot2_bf16(P[h], d6, o[6]); o[7] = dot2_bf16(P[h], d7, o[7]);
      }
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
        const uint32_t a0 = code8x2_to_bf16x2<CDT, false>(f.v[0][i]);
        const uint32_t b0 = code8x2_to_bf16x2<CDT, false>(f.v[1][i]);
        const uint32_t a1 = code8x2_to_bf16x2<CDT, true>(f.v[0][i]);
        const uint32_t b1 = code8x2_to_bf16x2<CDT, true>(f.v[1][i]);
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
  return (k * 8 * L::CHUNK + c * L::CHUNK) * 8 / L::EBITS + w;
}

// ---------------------------------------------------------------------------
// Work decomposition (balanced, deterministic)
//
// A unit is one 16-token step of one (sequence, KV head group) segment, a
// group being the hw consecutive KV heads that the hw waves of a workgroup
// take; units are ordered by (sequence, head group, step).  A segment with
// steps also counts ov start-up units ahead of its steps (decode_seg_ov: 2
// for 32- and 16-bit caches, 6 for 8- and 4-bit ones): a piece of a segment
// loads its queries, fills its load pipeline and stores its partial, which is
// worth more steps where steps carry fewer bytes (on the long-tail step with
// 8-bit codes, each further sequence a workgroup touched added 6.5 us to its
// 280 us, and the launch lasted as long as its workgroups with 5-8 sequences;
// split kernel with 0/2/4/6/8 start-up units, one box: int8 334.9/324.9/
// 320.2/315.5/313.9 us, int4 259.1/253.0/249.6/249.5/250.0 us, bf16
// 604.1/594.5/596.6/598.8/598.8 us, Llama-3 211.5/209.6/209.8/209.6/211.9 us).
// The split kernel writes ov into the workspace header for the merge.  With U units and W resident workgroups, workgroup w processes
// units [floor(w U / W), floor((w+1) U / W)): every workgroup gets the same
// time's worth of work, whatever the mix of context lengths; a range that
// holds only start-up units of a segment computes nothing there.  Each wave emits one partial (m, l, O) for every
// segment piece it covers; the piece of workgroup w in segment g is stored in
// slot w + g (one entry per wave of the group), which is unique because both
// workgroup and segment boundaries are increasing along the unit order.  The
// merge kernel finds the workgroups covering a segment from its unit range.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int steps_of(int ctx) { return ctx > 0 ? (ctx + 15) >> 4 : 0; }
// units of a segment in the split: its steps and ov start-up units
__host__ __device__ __forceinline__ int units_of(int ctx, int ov) {
  return ctx > 0 ? ((ctx + 15) >> 4) + ov : 0;
}

// Both quotients are taken in double precision instead of 64-bit integer
// division (a long scalar sequence, on the merge kernel's critical path).  They
// are exact: with U < 2^31 units and W <= 2^20 workgroups the numerators are
// below 2^53 (exact doubles), and a quotient that is not an integer lies at
// least 1/W (1/U) from the next integer, more than the rounding error of the
// division (half an ulp of a quotient below 2^31 (2^20), at most 2^-23
// (2^-33)), so the floor of the rounded quotient is the integer quotient.
//
// The split is weighted by XCD.  Workgroup w runs on XCD w % 8 (the launch
// hands workgroups to the eight XCDs round robin), and on MI355X the
// workgroups of the odd XCDs took 5-8% longer than those of the even ones for
// the same units (decode split kernel, Llama-3 and long-tail int8 steps, four
// boxes: odd/even time 1.052-1.084).  With W a multiple of 8 (and at most 2^17,
// which keeps the quotients below exact), a workgroup of an odd XCD takes
// DEC_WT_ODD / DEC_WT_EVEN of an even one's share: workgroup w begins at unit
// floor(U S(w) / S(W)), S(w) the weights of workgroups [0, w).  The weights
// move split points only.  Exactness with weights: U S(w) < 2^31 * 2^21.1,
// below 2^53, and a non-integer quotient lies at least 1 / S(W) >= 2^-21.1
// from an integer, more than the rounding error (2^-22).
constexpr int DEC_WT_EVEN = 17, DEC_WT_ODD = 16;
__device__ __forceinline__ bool dec_weighted(int W) { return (W & 7) == 0 && W <= (1 << 17); }
__device__ __forceinline__ int64_t dec_wsum(int w) {
  return (int64_t)DEC_WT_EVEN * ((w + 1) >> 1) + (int64_t)DEC_WT_ODD * (w >> 1);
}
__device__ __forceinline__ int64_t wave_begin(int w, int64_t U, int W) {
  if (dec_weighted(W))
    return (int64_t)__builtin_floor((double)U * (double)dec_wsum(w) / (double)dec_wsum(W));
  return (int64_t)__builtin_floor((double)w * (double)U / (double)W);
}
// the workgroup whose unit range holds unit x (0 <= x < U); with weights the
// unweighted owner is at most one workgroup off, and is corrected
__device__ __forceinline__ int wave_of(int64_t x, int64_t U, int W) {
  int w = (int)__builtin_floor(((double)(x + 1) * (double)W - 1.0) / (double)U);
  if (!dec_weighted(W)) return w;
  w = min(max(w, 0), W - 1);
  while (w > 0 && wave_begin(w, U, W) > x) --w;
  while (w + 1 < W && wave_begin(w + 1, U, W) <= x) ++w;
  return w;
}

// Units of the sequences before `s` (pre) and in total (all), one pass of the
// wave over context_lens (nhg = head groups per sequence).
__device__ __forceinline__ void unit_counts(const int32_t* __restrict__ ctx, int num_seqs, int nhg,
                                            int ov, int s, int* pre, int* all) {
  int a = 0, b = 0;
  for (int i = threadIdx.x & 63; i < num_seqs; i += 64) {
    const int v = nhg * units_of(ctx[i], ov);
    b += v;
    if (i < s) a += v;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
  }
  // the reductions leave the same value in every lane: make it wave-uniform
  *pre = __builtin_amdgcn_readfirstlane(a);
  *all = __builtin_amdgcn_readfirstlane(b);
}

// The sequence holding unit x (0 <= x < U) and the units before it.
__device__ __forceinline__ void locate_unit(const int32_t* __restrict__ ctx, int num_seqs, int nhg,
                                            int ov, int x, int* seq, int* before) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    const int i = base + lane;
    const int v = i < num_seqs ? nhg * units_of(ctx[i], ov) : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const uint64_t hit = __ballot(carry + incl > x);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      *seq = __builtin_amdgcn_readfirstlane(base + l);
      *before = __builtin_amdgcn_readfirstlane(carry + __shfl(incl - v, l, 64));
      return;
    }
    carry = __builtin_amdgcn_readfirstlane(carry + __shfl(incl, 63, 64));
  }
  *seq = num_seqs - 1;   // not reached for x < U
  *before = carry;
}

// The start of workgroup w: the total units U, its range [u0, u1) and, when
// the range is not empty, the sequence s holding u0 and the units before s.
// Up to 64 * DEC_CTX_REGS sequences, context_lens is read in one round of
// loads held in registers (every load issued before the first is used), and
// U and s come from those registers; longer batches take the two passes of
// unit_counts and locate_unit (one round of loads per 64 sequences each).
constexpr int DEC_CTX_REGS = 4;
__device__ __forceinline__ void wg_plan(const int32_t* __restrict__ ctx, int num_seqs, int nhg,
                                        int ov, int w, int W, int* U, int64_t* u0, int64_t* u1,
                                        int* seq, int* before) {
  if (num_seqs > 64 * DEC_CTX_REGS) {
    int pre;
    unit_counts(ctx, num_seqs, nhg, ov, 0, &pre, U);
    *u0 = wave_begin(w, *U, W);
    *u1 = wave_begin(w + 1, *U, W);
    if (*u0 < *u1) locate_unit(ctx, num_seqs, nhg, ov, (int)*u0, seq, before);
    return;
  }
  const int lane = threadIdx.x & 63;
  int v[DEC_CTX_REGS];
#pragma unroll
  for (int c = 0; c < DEC_CTX_REGS; ++c) {
    const int i = 64 * c + lane;
    v[c] = i < num_seqs ? ctx[i] : 0;
  }
  int tot = 0;
#pragma unroll
  for (int c = 0; c < DEC_CTX_REGS; ++c) {
    v[c] = nhg * units_of(v[c], ov);
    tot += v[c];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
  *U = __builtin_amdgcn_readfirstlane(tot);
  *u0 = wave_begin(w, *U, W);
  *u1 = wave_begin(w + 1, *U, W);
  if (*u0 >= *u1) return;
  const int x = (int)*u0;
  int carry = 0;
#pragma unroll
  for (int c = 0; c < DEC_CTX_REGS; ++c) {
    int incl = v[c];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const uint64_t hit = __ballot(carry + incl > x);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      *seq = __builtin_amdgcn_readfirstlane(64 * c + l);
      *before = __builtin_amdgcn_readfirstlane(carry + __shfl(incl - v[c], l, 64));
      return;
    }
    carry = __builtin_amdgcn_readfirstlane(carry + __shfl(incl, 63, 64));
  }
  *seq = num_seqs - 1;   // not reached for x < U
  *before = carry;
}

// Steps [st0, st1) of segment (s, kvh): online softmax, then the partial of
// this piece into entry `slot` of the partial arrays.
template <int CDT, int HD, int G, int NBUF>
__device__ __forceinline__ void decode_run(const DecodeArgs& a, int s, int kvh, int st0, int st1,
                                           int64_t slot) {
  using L = DecodeLayout<CDT, HD>;
  const int lane = threadIdx.x & 63;
  const int lane_g = lane >> 3, lane_c = lane & 7;
  const int ctx = uniform_load(a.context_lens, s);
  const int begin = st0 * 16;
  const int end = min(ctx, st1 * 16);
  const int n_q = a.n_kv * G;

  DecodeState<CDT, HD, G> st;
  // query fragment: the same dims as this lane's K/V elements
  if constexpr (CDT == PA_INT4) {
    // times the key scale of each channel (folded into the query, rounded to
    // bf16), packed as the pairs (0,2) (4,6) (1,3) (5,7) of each 8 dims
    const int d0 = lane_dim<L>(lane_c, 0);
    const float* ks = a.k_ch_scale + (int64_t)kvh * HD + d0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint8_t* p = a.q + (((int64_t)s * n_q + (int64_t)kvh * G + h) * HD + d0) * 2;
#pragma unroll
      for (int i = 0; i < L::DW; ++i) {
        const uint4 x = *(const uint4*)(p + 16 * i);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16lo_f32(w[e]) * ks[8 * i + 2 * e];
          f[2 * e + 1] = bf16hi_f32(w[e]) * ks[8 * i + 2 * e + 1];
        }
        st.q[h][4 * i + 0] = pack_bf16(f[0], f[2]);
        st.q[h][4 * i + 1] = pack_bf16(f[4], f[6]);
        st.q[h][4 * i + 2] = pack_bf16(f[1], f[3]);
        st.q[h][4 * i + 3] = pack_bf16(f[5], f[7]);
      }
      st.m[h] = -1e30f;
      st.l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < L::DPL; ++e) st.o[h][e] = 0.0f;
    }
  } else {
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

  const int trow = a.table_row ? uniform_load(a.table_row, s) : s;
  const int32_t* table = a.block_tables + (int64_t)trow * a.max_blocks;
  const int lane_byte = lane_c * L::CHUNK;
  const float c = a.score_scale;

  if (a.block_size >= 16) {
    const int n_full = (end - begin) >> 4;
    const int tail = begin + (n_full << 4);
    if (tail < end) {               // the ragged last step of the sequence, masked, first
      Frag<L> t;
      load_step<L>(t, a, table, tail, end, kvh, lane_g, lane_byte);
      process_step<CDT, HD, G, true>(st, t, c);
    }
    if (n_full > 0) {
      // NBUF fragments: NBUF - 1 steps in flight while one is computed.  Loads
      // past the last step go through an empty descriptor, so the loop body
      // always issues the same loads and the waits stay tight.
      const uint32_t lane_off = (uint32_t)(kvh * L::ROW + lane_byte + lane_g * (int)a.tok_stride);
      Frag<L> buf[NBUF];
#pragma unroll
      for (int d = 0; d < NBUF - 1; ++d)
        load_full_step<L>(buf[d], a, table, begin + 16 * min(d, n_full - 1), lane_off, d < n_full,
                          kvh, lane_g);
      int i = 0;
      for (; i + NBUF <= n_full; i += NBUF) {   // every path issues NBUF step loads
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          const int pf = i + u + NBUF - 1;
          load_full_step<L>(buf[(u + NBUF - 1) % NBUF], a, table, begin + 16 * min(pf, n_full - 1),
                            lane_off, pf < n_full, kvh, lane_g);
          process_step<CDT, HD, G, false>(st, buf[u], c);
        }
      }
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u) {       // the last n_full % NBUF steps
        const int pf = i + u + NBUF - 1;
        load_full_step<L>(buf[(u + NBUF - 1) % NBUF], a, table, begin + 16 * min(pf, n_full - 1),
                          lane_off, pf < n_full, kvh, lane_g);
        if (i + u < n_full) process_step<CDT, HD, G, false>(st, buf[u], c);
      }
    }
  } else {
    // blocks smaller than a step: per-lane table lookups, masked loads
    Frag<L> fa, fb;
    int base = begin;
    load_step<L>(fa, a, table, base, end, kvh, lane_g, lane_byte);
    while (true) {
      const int nb = base + 16;
      if (nb < end) load_step<L>(fb, a, table, nb, end, kvh, lane_g, lane_byte);
      process_step<CDT, HD, G, true>(st, fa, c);
      if (nb >= end) break;
      const int nn = nb + 16;
      if (nn < end) load_step<L>(fa, a, table, nn, end, kvh, lane_g, lane_byte);
      process_step<CDT, HD, G, true>(st, fb, c);
      if (nn >= end) break;
      base = nn;
    }
  }

  // merge the 8 lane groups (lane-local softmax states) of this wave
  float* out_o = a.part_o + slot * G * HD;
  float* out_ml = a.part_ml + slot * G * 2;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = max_over_groups(st.m[h]);
    const float w = fast_exp2(st.m[h] - M);
    const float lsum = sum_over_groups(st.l[h] * w);
    float ov[L::DPL];
#pragma unroll
    for (int e = 0; e < L::DPL; ++e) ov[e] = sum_over_groups(st.o[h][e] * w);
    if (lane_g == h) {   // lanes of group h store head h
      float* dst = out_o + h * HD;
#pragma unroll
      for (int k = 0; k < L::NCHUNK; ++k) {
        const int d0 = lane_dim<L>(lane_c, k * L::EPC);
#pragma unroll
        for (int i = 0; i < L::EPC; i += 4)
          *(float4*)(dst + d0 + i) = make_float4(ov[k * L::EPC + i], ov[k * L::EPC + i + 1],
                                                 ov[k * L::EPC + i + 2], ov[k * L::EPC + i + 3]);
      }
      if (lane_c == 0) *(float2*)(out_ml + 2 * h) = make_float2(M, lsum);
    }
  }
}

// hw waves per workgroup; workgroup w walks its unit range segment by
// segment, wave i of the group on KV head hg * hw + i of head group hg.
template <int CDT, int HD, int G, int NBUF>
__global__ __launch_bounds__(64 * max_hw(CDT, G)) void decode_split_kernel(DecodeArgs a) {
  const int w = blockIdx.x;
  const int W = a.num_wgs;
  const int wv = threadIdx.x >> 6;
  constexpr int OV = decode_seg_ov(CDT);
  int U, s = 0, before = 0;
  int64_t u0, u1;
  wg_plan(a.context_lens, a.num_seqs, a.nhg, OV, w, W, &U, &u0, &u1, &s, &before);
  if (w == 0 && threadIdx.x == 0) *(int4*)a.header = make_int4(W, a.hw, OV, U);   // for the merge
  if (u0 >= u1) return;
  const int len0 = units_of(uniform_load(a.context_lens, s), OV);
  const int r = (int)u0 - before;
  int hg = r / len0;
  int off = r % len0;                  // unit offset in the segment
  int64_t u = u0;
  while (true) {
    const int len = units_of(uniform_load(a.context_lens, s), OV);
    const int end = (int)min((int64_t)len, off + (u1 - u));
    const int sb = max(off - OV, 0), se = max(end - OV, 0);   // steps
    const int64_t g = (int64_t)s * a.nhg + hg;
    if (se > sb) {
      decode_run<CDT, HD, G, NBUF>(a, s, hg * a.hw + wv, sb, se, (w + g) * a.hw + wv);
      if (threadIdx.x == 0) {   // the merge reads the segment's pieces from these
        if (sb == 0) a.seg_w[2 * g] = w;
        if (se == len - OV) a.seg_w[2 * g + 1] = w;
      }
    }
    u += end - off;
    if (u >= u1) break;
    off = 0;
    if (++hg == a.nhg) {               // next sequence that has tokens
      hg = 0;
      do { ++s; } while (steps_of(uniform_load(a.context_lens, s)) == 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path (block_size >= 16).  The same work split, pieces and
// partial format as above; inside a wave both products run on MFMA:
//   * S^T = K Q'^T with v_mfma_f32_16x16x32_bf16: lane l = (j = l / 16,
//     r = l % 16) holds token r of the 16-token step, dims [j HD/4, (j+1) HD/4)
//     of K as the A operand (its natural layout: one contiguous piece of the
//     token's row per lane) and, as the B operand, the same dims of query head
//     r (zero for r >= G).  The result gives each lane tokens 4j .. 4j+3 of
//     head column r.
//   * O = P V with v_mfma_f32_16x16x16_bf16: those four weights are already the
//     A operand (row = head r, k = tokens 4j .. 4j+3).  V is converted to bf16,
//     written as rows to this wave's slice of LDS, and read back transposed with
//     ds_read_b64_tr_b16, which hands lane (j, r) tokens 4j .. 4j+3 of one dim:
//     the B operand.  The output gives each lane heads 4j .. 4j+3 of dim r of
//     each 16-dim block.
// The softmax runs per head column: the four lanes of a column (j = 0..3)
// agree on its running max with two exchanges per step, and the max moves only
// when a tile max exceeds it by more than DMF_SLACK (base-2 units), as in the
// chunked-prefill kernel.  This takes the two products off the vector ALU,
// which otherwise bounds the 8- and 4-bit caches (their codes must be widened
// to bf16 either way).
// Loads come in one of two forms:
//   * per head: each wave loads its own head's rows, 64 contiguous bytes per
//     token (16 tokens per instruction, one token stride apart);
//   * staged (STAGED): the workgroup's waves load the step's rows of all its
//     heads together, each instruction covering 1 KiB of whole token rows in
//     order, write them to a double-buffered LDS stage (16-byte chunks XOR-
//     swizzled by token, so its writes and reads meet no bank conflicts)
//     and each wave reads its head's pieces back from there.  One barrier per
//     step; a step is written to the stage one step before it is read.  Long
//     runs of whole rows stream from HBM faster than per-head pieces.
// ---------------------------------------------------------------------------
typedef __bf16 mf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef short mf_s4_t __attribute__((ext_vector_type(4)));
typedef float mf_f32x4_t __attribute__((ext_vector_type(4)));
constexpr float DMF_SLACK = 8.0f;

template <int CDT, int HD>
struct MfLayout {
  static constexpr int EBITS = DecodeLayout<CDT, HD>::EBITS;
  static constexpr int ROW = HD * EBITS / 8;     // bytes of one (token, head) row
  static constexpr int DPJ = HD / 4;             // dims per lane group j
  static constexpr int JB = DPJ * EBITS / 8;     // bytes per lane per token
  static constexpr int KW = JB / 4;              // dwords per lane per token
  // A lane's bytes of a token row come in NP pieces of PS bytes: piece k of
  // lane group j at byte (j + 4k) PS, so the four lanes of a token read PS * 4
  // contiguous bytes per load instruction.
  static constexpr int PS = JB < 16 ? JB : 16;
  static constexpr int NP = JB / PS;
  static constexpr int DPP = PS * 8 / EBITS;     // dims per piece
  static constexpr int NT = HD / 32;             // QK MFMAs (16x16x32) per step
  static constexpr int NB = HD / 16;             // PV MFMAs (16x16x16) per step
  static constexpr int VROW = HD * 2;            // LDS bytes per token row of V (bf16)
  static constexpr int WAVE_LDS = 16 * VROW;
  // staged loads: 16-byte chunks per lane per step, and the bytes of one
  // tensor's stage (16 tokens of up to DECODE_MAX_HW heads)
  static constexpr int LIN = ROW / 64;
  static constexpr int STAGE = 16 * DECODE_MAX_HW * ROW;
};

// The staged form applies to 16- and 8-bit codes when a lane's piece is 16
// bytes and a head group's token row is a whole number of 16-chunk (256-byte)
// swizzle groups.  On the long-tail step it took int8 from 364 to 327 us and
// fp8 from 356 (vector kernel) to 326 us.  int4 keeps per-head loads: its
// steps carry the most vector work per byte (the nibble widening), and a
// barrier per step that keeps the 8 waves in the same phase cost more than the
// longer runs gained (285 against 251 us).
template <int CDT, int HD>
__host__ __device__ constexpr bool mf_stageable_layout() {
  return (MfLayout<CDT, HD>::EBITS == 8 || MfLayout<CDT, HD>::EBITS == 16) &&
         MfLayout<CDT, HD>::PS == 16 && MfLayout<CDT, HD>::LIN >= 1;
}
__host__ __device__ inline bool mf_staged_ok(int row_bytes, int hw) {
  return row_bytes >= 64 && (hw * row_bytes) % 256 == 0;
}

#ifndef DECODE_MF_AUX
#define DECODE_MF_AUX DECODE_LOAD_AUX
#endif
// LDS bank groups, as the SQ bank-conflict counter shows them on gfx950: a
// 16-byte access (ds_read_b128 / ds_write_b128) is served 8 lanes at a time,
// free of conflicts when the 8 chunks differ in bits 4..6 of their addresses
// (a 128-byte window); ds_read_b64_tr_b16 is served 32 lanes at a time, free
// when the 32 pieces differ in bits 3..7 (a 256-byte window).
//
// Rows of 16 tokens in LDS (the load stage, a wave's V slice) keep 16-byte
// chunk c of token row t at chunk c ^ row_g(t).  Over any 8 consecutive rows
// row_g takes 8 different values mod 8 (so one chunk of 8 rows, the slice
// writes and the stage's per-head reads, fills a 128-byte window) and 8
// different values of row_g / 2 (so a 32-byte pair of chunks of 8 rows, the
// transposed reads, fills a 256-byte window); whole 128-byte runs of one row
// (the stage writes) stay whole.  (t ^ c alone left two rows per pair of
// chunks in the transposed reads; t << 1 alone, two rows per window in the
// slice writes.)
__device__ __forceinline__ int row_g(int t) { return ((t & 7) << 1) | ((t >> 2) & 1); }
// A wave's V slice (16 token rows of bf16): rows of 256 bytes (head_dim 128)
// take row_g; rows of 128 bytes (head_dim 64) sit two to a 256-byte window,
// so t & 7 spreads both kinds of access there.
template <int HD>
__device__ __forceinline__ int vslice_g(int t) {
  if constexpr (HD == 128) return row_g(t);
  else return t & 7;
}
template <int HD>
__device__ __forceinline__ uint32_t vslice_off(int t, int byte) {
  return (uint32_t)(t * 2 * HD + 16 * ((byte >> 4) ^ vslice_g<HD>(t)) + (byte & 15));
}

// First dim of the 8 dims that MFMA t of a step takes from lane group j.
template <class ML>
__device__ __forceinline__ int mf_dim0(int t, int j) {
  constexpr int CPP = ML::DPP / 8;   // 8-dim chunks per piece
  return (j + 4 * (t / CPP)) * ML::DPP + 8 * (t % CPP);
}

// One lane's K or V codes of one token: NP pieces (see MfLayout).
template <class ML>
__device__ __forceinline__ void mf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                        uint32_t (&d)[ML::KW]) {
  static_assert(ML::PS == 16 || ML::PS == 8, "lane pieces of 8 or 16 bytes");
#pragma unroll
  for (int k = 0; k < ML::NP; ++k) {
    if constexpr (ML::PS == 8) {
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 32 * k, 0, DECODE_MF_AUX);
      d[2 * k + 0] = x.x; d[2 * k + 1] = x.y;
    } else {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 64 * k, 0, DECODE_MF_AUX);
      d[4 * k + 0] = x.x; d[4 * k + 1] = x.y; d[4 * k + 2] = x.z; d[4 * k + 3] = x.w;
    }
  }
}

template <class ML>
struct MfFrag {
  uint32_t k[ML::KW];
  uint32_t v[ML::KW];
  float vs[4];   // INT4: value scales of tokens 4j .. 4j+3
  int nb;        // staged form: block id of the step NBUF steps later
};

// The loads of one step: tokens [base, base + 16) of the sequence, all in one
// block (block_size >= 16).  Tokens at or past `end` read as zeros (the
// descriptor covers only the valid rows), as does a step with live == false.
template <int CDT, class ML>
__device__ __forceinline__ void mf_load_step(MfFrag<ML>& f, const DecodeArgs& a, int blk,
                                             int base, int end, uint32_t lane_off, bool live,
                                             int kvh, int j) {
  const int64_t tok0 = (int64_t)blk * a.block_size + (base & (a.block_size - 1));
  const int n = live ? min(16, end - base) : 0;
  const int32_t bytes = n * (int32_t)a.tok_stride;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k_cache + tok0 * a.tok_stride, bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v_cache + tok0 * a.tok_stride, bytes);
  mf_load<ML>(kr, lane_off, f.k);
  mf_load<ML>(vr, lane_off, f.v);
  if constexpr (CDT == PA_INT4) {   // tokens 4j .. 4j+3: adjacent in the scale pool
    const float4 x = *(const float4*)(a.v_tok_scale +
                                      ((int64_t)blk * a.n_kv + kvh) * a.block_size +
                                      (base & (a.block_size - 1)) + 4 * j);
    f.vs[0] = x.x; f.vs[1] = x.y; f.vs[2] = x.z; f.vs[3] = x.w;   // masked where used
  }
}

// Eight dims of K as an MFMA operand (bf16), from dwords d[w0 ..] of the lane's
// codes.  INT4 pairs come out as dims (0,2) (4,6) (1,3) (5,7); the query was
// packed in the same order.
template <int CDT>
__device__ __forceinline__ mf_bf16x8_t mf_k8(const uint32_t* d) {
  uint32_t w[4];
  if constexpr (CDT == PA_BF16) {
    w[0] = d[0]; w[1] = d[1]; w[2] = d[2]; w[3] = d[3];
  } else if constexpr (CDT == PA_INT4) {
    const uint32_t lo = int4_lo_as_e4m3(d[0]), hi = int4_hi_as_e4m3(d[0]);
    w[0] = int4e4m3_to_bf16x2<false>(lo); w[1] = int4e4m3_to_bf16x2<true>(lo);
    w[2] = int4e4m3_to_bf16x2<false>(hi); w[3] = int4e4m3_to_bf16x2<true>(hi);
  } else {
    w[0] = code8x2_to_bf16x2<CDT, false>(d[0]); w[1] = code8x2_to_bf16x2<CDT, true>(d[0]);
    w[2] = code8x2_to_bf16x2<CDT, false>(d[1]); w[3] = code8x2_to_bf16x2<CDT, true>(d[1]);
  }
  return __builtin_bit_cast(mf_bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}
// dwords of the lane's codes per 8 dims
template <int CDT>
constexpr int mf_dw8() { return CDT == PA_BF16 ? 4 : CDT == PA_INT4 ? 1 : 2; }

// LDS column of dim c of a token row: INT4 rows keep each 8 dims in the
// converter's order 0 2 4 6 1 3 5 7, the others in order.
template <int CDT>
__device__ __forceinline__ int mf_dim_of_col(int c) {
  if constexpr (CDT == PA_INT4) {
    const int p = c & 7;
    return (c & ~7) + (p < 4 ? 2 * p : 2 * (p - 4) + 1);
  } else {
    return c;
  }
}

// Staged loads: the lane's linear chunks of a step (global offsets from the
// head group's row start of the step's first token), where they go in the
// stage, and where the lane's own pieces are read back.
template <class ML>
struct MfStageMap {
  uint32_t goff[ML::LIN];
  uint32_t wpos[ML::LIN];
  uint32_t rpos[ML::NP];
};

template <class ML>
__device__ __forceinline__ MfStageMap<ML> mf_stage_map(const DecodeArgs& a, int wv, int lane) {
  MfStageMap<ML> m;
  const int rc_log2 = __builtin_ctz((unsigned)(a.hw * ML::ROW / 16));   // chunks per token row
  const int rc = 1 << rc_log2;
  const int j = lane >> 4, r = lane & 15;
#pragma unroll
  for (int k = 0; k < ML::LIN; ++k) {
    const int q = (k * a.hw + wv) * 64 + lane;   // chunk of the step, in memory order
    const int t = q >> rc_log2, c = q & (rc - 1);
    m.goff[k] = (uint32_t)(t * (int)a.tok_stride + 16 * c);
    m.wpos[k] = (uint32_t)(16 * (t * rc + (c ^ row_g(t))));
  }
#pragma unroll
  for (int k = 0; k < ML::NP; ++k) {
    const int c = wv * (ML::ROW / 16) + j + 4 * k;   // piece k of lane group j, head wv
    m.rpos[k] = (uint32_t)(16 * (r * rc + (c ^ row_g(r))));
  }
  return m;
}

// LDS-only barrier: the stage's writes are visible to the workgroup after it,
// and global loads in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CDT, int HD, int G, int NBUF, bool STAGED, bool APPEND>
__device__ __forceinline__ void decode_run_mf(const DecodeArgs& a, int s, int kvh, int st0,
                                              int st1, int64_t slot, uint8_t* vl, int wv,
                                              uint8_t* stage) {
  using ML = MfLayout<CDT, HD>;
  constexpr int DW8 = mf_dw8<CDT>();
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, r = lane & 15;
  const int ctx = uniform_load(a.context_lens, s);
  const int begin = st0 * 16;
  const int end = min(ctx, st1 * 16);
  const int n_q = a.n_kv * G;
  const float c = a.score_scale;

  // B operand of QK: head r, dims j DPJ + 8t + e (INT4: times the key scale of
  // the channel, in the converter's pair order); zero for r >= G
  mf_bf16x8_t qb[ML::NT];
  {
    const int h = r < G ? r : 0;
    const int64_t qr = a.row_map ? uniform_load(a.row_map, s) : s;
    const uint8_t* qp = a.q + (qr * n_q + (int64_t)kvh * G + h) * HD * 2;
#pragma unroll
    for (int t = 0; t < ML::NT; ++t) {
      const int d0 = mf_dim0<ML>(t, j);
      const uint4 x = *(const uint4*)(qp + 2 * d0);
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
      if constexpr (CDT == PA_INT4) {
        const float* ks = a.k_ch_scale + (int64_t)kvh * HD + d0;
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16lo_f32(w[e]) * ks[2 * e];
          f[2 * e + 1] = bf16hi_f32(w[e]) * ks[2 * e + 1];
        }
        w[0] = pack_bf16(f[0], f[2]); w[1] = pack_bf16(f[4], f[6]);
        w[2] = pack_bf16(f[1], f[3]); w[3] = pack_bf16(f[5], f[7]);
      }
      if (r >= G) w[0] = w[1] = w[2] = w[3] = 0u;
      qb[t] = __builtin_bit_cast(mf_bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  mf_f32x4_t acc[ML::NB];
#pragma unroll
  for (int b = 0; b < ML::NB; ++b) acc[b] = mf_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -1e30f;     // running max of head column r (base-2 units, scaled)
  float lp = 0.0f;      // this lane's share of l for column r

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const uint32_t lane_off = (uint32_t)(r * (int)a.tok_stride + kvh * ML::ROW + j * ML::PS);
  // Block ids, 64 at a time in a vector register (lane i: table entry c0 + i),
  // the next 64 loaded a chunk ahead: a step picks its id with a lane read and
  // never waits on a table load (a scalar load would make every step wait for
  // its latency, together with the wave's LDS traffic).
  const int jlast = min((end - 1) >> a.bs_log2, a.max_blocks - 1);
  auto tload = [&](int c0) -> int {
    const int jj = c0 + lane;
    return jj <= jlast ? table[jj] : 0;
  };
  int c0 = begin >> a.bs_log2;
  int tA = tload(c0), tB = tload(c0 + 64);
  auto block_at = [&](int base) -> int {   // base: wave-uniform, non-decreasing
    const int jb = base >> a.bs_log2;
    while (jb >= c0 + 64) {
      c0 += 64;
      tA = tB;
      tB = tload(c0 + 64);
    }
    const int blk = __builtin_amdgcn_readlane(tA, jb - c0);
    return (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
  };

  // bf16 rows staged in LDS are already the V operand's rows: its transposed
  // reads go to the stage directly (lane (j, r): token 4j + r / 4, the 8 bytes
  // at 32 b + 8 (r % 4) of the head's row, through the stage's swizzle), and
  // the wave needs no V slice of its own.
  constexpr bool VDIRECT = STAGED && CDT == PA_BF16;
  uint32_t vrd[VDIRECT ? ML::NB : 1];
  // otherwise the slice's write offsets (token r, this lane's dims of MFMA t)
  // and transposed-read offsets (tokens 4j .. 4j+3, dims 16 b + r)
  uint32_t vwo[VDIRECT ? 1 : ML::NT], vro[VDIRECT ? 1 : ML::NB];
  if constexpr (!VDIRECT) {
#pragma unroll
    for (int t = 0; t < ML::NT; ++t) vwo[t] = vslice_off<HD>(r, 2 * mf_dim0<ML>(t, j));
#pragma unroll
    for (int b = 0; b < ML::NB; ++b) vro[b] = vslice_off<HD>(4 * j + (r >> 2), 32 * b + 8 * (r & 3));
  }
  if constexpr (VDIRECT) {
    constexpr int CPR = ML::ROW / 16;        // 16-byte chunks of one head's row
    const int rc = a.hw * CPR;
    const int t = 4 * j + (r >> 2);
#pragma unroll
    for (int b = 0; b < ML::NB; ++b) {
      const int c = wv * CPR + 2 * b + ((r >> 1) & 1);   // chunk of bytes 32 b + 8 (r % 4)
      vrd[b] = (uint32_t)(16 * (t * rc + (c ^ row_g(t))) + 8 * (r & 1));
    }
  }

  auto step = [&](const uint32_t* fk, const uint32_t* fv, const float* fvs, int base,
                  const uint8_t* vsrc) {
    // S^T: tokens 4j .. 4j+3 of head column r
    mf_f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < ML::NT; ++t)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mf_k8<CDT>(fk + DW8 * t), qb[t], sc, 0, 0, 0);
    // V rows (bf16) into this wave's LDS slice: token r, this lane's dims
    if constexpr (!VDIRECT) {
#pragma unroll
      for (int t = 0; t < ML::NT; ++t) {
        const mf_bf16x8_t v8 = mf_k8<CDT>(fv + DW8 * t);
        *(uint4*)(vl + vwo[t]) = __builtin_bit_cast(uint4, v8);
      }
    }
    // softmax of column r over the step's 16 tokens
    const int nvalid = end - base;   // >= 1
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * j + i < nvalid) ? sc[i] * c : -INFINITY;
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__any(tmax > m + DMF_SLACK)) {   // wave-uniform: rescale to the new max
      const float mn = fmaxf(m, tmax);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lp *= alpha;
      // rows 4j+i of O belong to head column 4j+i; whole-vector products keep
      // each accumulator one register tuple
      const mf_f32x4_t av = {__shfl(alpha, 4 * j + 0, 64), __shfl(alpha, 4 * j + 1, 64),
                             __shfl(alpha, 4 * j + 2, 64), __shfl(alpha, 4 * j + 3, 64)};
#pragma unroll
      for (int b = 0; b < ML::NB; ++b) acc[b] *= av;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m);
    uint32_t P0, P1;
    if constexpr (CDT == PA_INT4) {     // value scale of each token into its weight
      lp += (p[0] + p[1]) + (p[2] + p[3]);
      float sv[4];                      // scales of tokens past the end read as 0
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (4 * j + i < nvalid) ? fvs[i] : 0.0f;
      P0 = pack_bf16(p[0] * sv[0], p[1] * sv[1]);
      P1 = pack_bf16(p[2] * sv[2], p[3] * sv[3]);
    } else {                            // l from the rounded weights
      P0 = pack_bf16(p[0], p[1]);
      P1 = pack_bf16(p[2], p[3]);
      lp = dot2_bf16(P0, 0x3F803F80u, lp);
      lp = dot2_bf16(P1, 0x3F803F80u, lp);
    }
    const mf_s4_t pa4 = __builtin_bit_cast(mf_s4_t, make_uint2(P0, P1));
    // V^T blocks: lane (j, r) gets tokens 4j .. 4j+3 of LDS column 16 b + r
#pragma unroll
    for (int b = 0; b < ML::NB; ++b) {
      const uint8_t* src;
      if constexpr (VDIRECT) src = vsrc + vrd[b];
      else src = vl + vro[b];
      const mf_s4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) mf_s4_t*)src);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa4, vb, acc[b], 0, 0, 0);
    }
  };

  // NBUF steps in flight; the same loads are issued on every path (past the
  // last step through an empty descriptor)
  const int nsteps = (end - begin + 15) >> 4;
  MfFrag<ML> buf[NBUF];
  if constexpr (!STAGED) {
    auto prefetch = [&](MfFrag<ML>& f, int pf) {
      const int base = begin + 16 * min(pf, nsteps - 1);
      mf_load_step<CDT, ML>(f, a, block_at(base), base, end, lane_off, pf < nsteps, kvh, j);
    };
#pragma unroll
    for (int d = 0; d < NBUF - 1; ++d) prefetch(buf[d], d);
    int i = 0;
    for (; i + NBUF <= nsteps; i += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        prefetch(buf[(u + NBUF - 1) % NBUF], i + u + NBUF - 1);
        step(buf[u].k, buf[u].v, buf[u].vs, begin + 16 * (i + u), nullptr);
      }
    }
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) {
      prefetch(buf[(u + NBUF - 1) % NBUF], i + u + NBUF - 1);
      if (i + u < nsteps) step(buf[u].k, buf[u].v, buf[u].vs, begin + 16 * (i + u), nullptr);
    }
  } else {
    // Step x is loaded into buf[x % NBUF], written to stage x & 1 while step
    // x - 1 is computed, and read back after that step's barrier.  Its block
    // id was loaded with step x - NBUF and travels in the same buffer; its
    // value scales (INT4, this wave's head) go to the stage with it.  No
    // loaded value outlives its buffer, so each wait covers exactly the step
    // being staged.
    const MfStageMap<ML> sm = mf_stage_map<ML>(a, wv, lane);
    // The appending decode: the run that reads the sequence's last token
    // (position ctx - 1, row tn of step xs) takes its K/V from k_new / v_new.
    // The lanes that stage that row's chunks encode them, write them to the
    // token's slot in the cache and, once the step is staged, over the stale
    // row in LDS; nothing else in the launch reads the slot.
    uint4 nk = make_uint4(0u, 0u, 0u, 0u), nv = nk;
    uint32_t npos = 0;
    bool nhave = false;
    int xs = -1;
    if constexpr (APPEND) {
      if (end == ctx) {
        const int p = ctx - 1;
        const int tn = p & 15;
        xs = (p - begin) >> 4;
        const int rc_log2 = __builtin_ctz((unsigned)(a.hw * ML::ROW / 16));
        const int rc = 1 << rc_log2;
        int cc = 0;
#pragma unroll
        for (int k = 0; k < ML::LIN; ++k) {
          const int q = (k * a.hw + wv) * 64 + lane;
          if ((q >> rc_log2) == tn) { nhave = true; cc = q & (rc - 1); }
        }
        const int64_t pslot = row_slot(table, a.max_blocks, a.block_size, a.bs_log2, p);
        if (nhave) {
          constexpr int EB = ML::EBITS / 8;
          const int64_t e0 = ((int64_t)s * a.n_kv + (kvh - wv)) * HD + 16 * cc / EB;
          const uint8_t* ksrc = a.k_new;
          const uint8_t* vsrc = a.v_new;
          nk = new_chunk<CDT>(ksrc, e0, a.src_f32 != 0, a.k_inv);
          nv = new_chunk<CDT>(vsrc, e0, a.src_f32 != 0, a.v_inv);
          npos = (uint32_t)(16 * (tn * rc + (cc ^ row_g(tn))));
          if (pslot >= 0 && pslot < (int64_t)a.num_blocks * a.block_size) {
            const int64_t off = pslot * a.tok_stride + (int64_t)(kvh - wv) * ML::ROW + 16 * cc;
            *(uint4*)((uint8_t*)a.k_cache + off) = nk;
            *(uint4*)((uint8_t*)a.v_cache + off) = nv;
          }
        }
        if (a.slots_out && kvh - wv == 0 && wv == 0 && lane == 0) a.slots_out[s] = pslot;
      }
    }
    float* vsl = (float*)(stage + 4 * ML::STAGE) + wv * 16 + 4 * j;   // + parity * 16 * DECODE_MAX_HW
    const int64_t hg_off = (int64_t)(kvh - wv) * ML::ROW;   // the head group's first row byte
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(table, (jlast + 1) * 4);
    auto table_at = [&](int pf) -> int {   // vector load, the same entry in every lane
      const int jb = (begin + 16 * min(pf, nsteps - 1)) >> a.bs_log2;
      return (int)__builtin_amdgcn_raw_buffer_load_b32(tr, (uint32_t)(4 * jb), 0, 0);
    };
    auto prefetch = [&](MfFrag<ML>& f, int pf, int blk) {
      const int base = begin + 16 * min(pf, nsteps - 1);
      blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
      const int64_t tok0 = (int64_t)blk * a.block_size + (base & (a.block_size - 1));
      const int n = pf < nsteps ? min(16, end - base) : 0;
      const int32_t bytes = n * (int32_t)a.tok_stride;
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k_cache + tok0 * a.tok_stride + hg_off, bytes);
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v_cache + tok0 * a.tok_stride + hg_off, bytes);
#pragma unroll
      for (int k = 0; k < ML::LIN; ++k) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(kr, sm.goff[k], 0, DECODE_MF_AUX);
        f.k[4 * k + 0] = x.x; f.k[4 * k + 1] = x.y; f.k[4 * k + 2] = x.z; f.k[4 * k + 3] = x.w;
        const u32x4_t y = __builtin_amdgcn_raw_buffer_load_b128(vr, sm.goff[k], 0, DECODE_MF_AUX);
        f.v[4 * k + 0] = y.x; f.v[4 * k + 1] = y.y; f.v[4 * k + 2] = y.z; f.v[4 * k + 3] = y.w;
      }
      if constexpr (CDT == PA_INT4) {   // this head's tokens 4j .. 4j+3 (masked where used)
        const float4 x = *(const float4*)(a.v_tok_scale +
                                          ((int64_t)blk * a.n_kv + kvh) * a.block_size +
                                          (base & (a.block_size - 1)) + 4 * j);
        f.vs[0] = x.x; f.vs[1] = x.y; f.vs[2] = x.z; f.vs[3] = x.w;
      }
      f.nb = table_at(pf + NBUF);
    };
    auto put = [&](const MfFrag<ML>& f, int x) {
      uint8_t* sk = stage + (x & 1) * 2 * ML::STAGE;
#pragma unroll
      for (int k = 0; k < ML::LIN; ++k) {
        *(uint4*)(sk + sm.wpos[k]) = make_uint4(f.k[4 * k], f.k[4 * k + 1], f.k[4 * k + 2], f.k[4 * k + 3]);
        *(uint4*)(sk + ML::STAGE + sm.wpos[k]) =
            make_uint4(f.v[4 * k], f.v[4 * k + 1], f.v[4 * k + 2], f.v[4 * k + 3]);
      }
      if constexpr (CDT == PA_INT4) {
        if (r == 0)
          *(float4*)(vsl + (x & 1) * 16 * DECODE_MAX_HW) = make_float4(f.vs[0], f.vs[1], f.vs[2], f.vs[3]);
      }
      if constexpr (APPEND) {   // the new token's row over the stale one (same lane, after it)
        if (x == xs && nhave) {
          *(uint4*)(sk + npos) = nk;
          *(uint4*)(sk + ML::STAGE + npos) = nv;
        }
      }
    };
    auto run = [&](int x) {
      const uint8_t* sk = stage + (x & 1) * 2 * ML::STAGE;
      uint32_t kc[ML::KW], vc[ML::KW];
#pragma unroll
      for (int k = 0; k < ML::NP; ++k) {
        const uint4 p = *(const uint4*)(sk + sm.rpos[k]);
        kc[4 * k] = p.x; kc[4 * k + 1] = p.y; kc[4 * k + 2] = p.z; kc[4 * k + 3] = p.w;
        if constexpr (!VDIRECT) {
          const uint4 q = *(const uint4*)(sk + ML::STAGE + sm.rpos[k]);
          vc[4 * k] = q.x; vc[4 * k + 1] = q.y; vc[4 * k + 2] = q.z; vc[4 * k + 3] = q.w;
        }
      }
      float vs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (CDT == PA_INT4) {
        const float4 t = *(const float4*)(vsl + (x & 1) * 16 * DECODE_MAX_HW);
        vs[0] = t.x; vs[1] = t.y; vs[2] = t.z; vs[3] = t.w;
      }
      step(kc, vc, vs, begin + 16 * x, sk + ML::STAGE);
    };
#pragma unroll
    for (int d = 0; d < NBUF; ++d) prefetch(buf[d], d, __builtin_amdgcn_readfirstlane(table_at(d)));
    put(buf[0], 0);
    lds_barrier();
    int i = 0;
    for (; i + NBUF <= nsteps; i += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        put(buf[(u + 1) % NBUF], i + u + 1);
        prefetch(buf[u], i + u + NBUF, __builtin_amdgcn_readfirstlane(buf[u].nb));
        run(i + u);
        lds_barrier();
      }
    }
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) {
      if (i + u < nsteps) {
        if (i + u + 1 < nsteps) put(buf[(u + 1) % NBUF], i + u + 1);
        run(i + u);
        lds_barrier();
      }
    }
  }

  // the piece's partial: l of column r summed over its four lanes; O rows 4j+i
  const float lsum = lp + __shfl_xor(lp, 16, 64);
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  float* out_o = a.part_o + slot * G * HD;
  float* out_ml = a.part_ml + slot * G * 2;
  const int dcol = mf_dim_of_col<CDT>(r);   // dim of LDS column r within each 16-block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * j + i;
    if (h < G) {
#pragma unroll
      for (int b = 0; b < ML::NB; ++b) out_o[h * HD + 16 * b + dcol] = acc[b][i];
    }
  }
  if (j == 0 && r < G) *(float2*)(out_ml + 2 * r) = make_float2(m, ltot);
}

// The matrix-core split kernel: the work loop of decode_split_kernel with
// decode_run_mf, and an LDS slice per wave for its V tile.
#ifndef DECODE_MF_MIN_WGS
#define DECODE_MF_MIN_WGS 1   // workgroups per CU the register budget must allow
#endif
template <int CDT, int HD, int G, int NBUF, bool STAGED, bool APPEND>
__global__ __launch_bounds__(64 * DECODE_MAX_HW, DECODE_MF_MIN_WGS) void decode_mfma_kernel(DecodeArgs a) {
  using ML = MfLayout<CDT, HD>;
  // per-wave V slices (none when bf16 V is read from the stage), then (staged)
  // two stages of K and V and the INT4 value scales of each stage's 16 tokens
  // per head
  constexpr int SLICES = (STAGED && CDT == PA_BF16) ? 0 : DECODE_MAX_HW * ML::WAVE_LDS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[SLICES +
      (STAGED ? 4 * ML::STAGE + (CDT == PA_INT4 ? 2 * DECODE_MAX_HW * 64 : 0) : 0)];
  const int w = blockIdx.x;
  const int W = a.num_wgs;
  const int wv = threadIdx.x >> 6;
  constexpr int OV = decode_seg_ov(CDT);
  int U, s = 0, before = 0;
  int64_t u0, u1;
  wg_plan(a.context_lens, a.num_seqs, a.nhg, OV, w, W, &U, &u0, &u1, &s, &before);
  if (w == 0 && threadIdx.x == 0) *(int4*)a.header = make_int4(W, a.hw, OV, U);   // for the merge
  if constexpr (APPEND) {   // sequences without tokens append nothing: slot -1
    if (w == 0 && a.slots_out)
      for (int i = threadIdx.x; i < a.num_seqs; i += blockDim.x)
        if (a.context_lens[i] <= 0) a.slots_out[i] = -1;
  }
  if (u0 >= u1) return;
  const int len0 = units_of(uniform_load(a.context_lens, s), OV);
  const int rr = (int)u0 - before;
  int hg = rr / len0;
  int off = rr % len0;                 // unit offset in the segment
  uint8_t* vl = lds + (SLICES ? wv * ML::WAVE_LDS : 0);
  auto run = [&](int rs, int rhg, int first, int last) {
    const int64_t slot = (int64_t)w + (int64_t)rs * a.nhg + rhg;
    decode_run_mf<CDT, HD, G, NBUF, STAGED, APPEND>(a, rs, rhg * a.hw + wv, first, last,
                                                    slot * a.hw + wv, vl, wv, lds + SLICES);
  };
  auto next_segment = [&]() {
    off = 0;
    if (++hg == a.nhg) {               // next sequence that has tokens
      hg = 0;
      do { ++s; } while (steps_of(uniform_load(a.context_lens, s)) == 0);
    }
  };
  int64_t u = u0;
  while (true) {
    const int len = units_of(uniform_load(a.context_lens, s), OV);
    const int end = (int)min((int64_t)len, off + (u1 - u));
    const int sb = max(off - OV, 0), se = max(end - OV, 0);   // steps
    if (se > sb) {
      run(s, hg, sb, se);
      if (threadIdx.x == 0) {   // the merge reads the segment's pieces from these
        const int64_t g = (int64_t)s * a.nhg + hg;
        if (sb == 0) a.seg_w[2 * g] = w;
        if (se == len - OV) a.seg_w[2 * g + 1] = w;
      }
    }
    u += end - off;
    if (u >= u1) break;
    next_segment();
  }
}

// One wave per (sequence, query head): combine the pieces' (m, l, O).
template <int HD, int G, bool OUT_BF16>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    void* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ header,
    const int32_t* __restrict__ seg_w, int num_seqs, int n_kv, float v_scale,
    const int32_t* __restrict__ row_map) {
  constexpr int DPT = HD / 64;   // dims per thread
  const int n_q = n_kv * G;
  const int hw = header[1];
  const int nhg = n_kv / hw;
  const int h = blockIdx.x % n_q;
  const int s = blockIdx.x / n_q;
  const int kvh = h / G, hl = h % G;
  const int hg = kvh / hw, wv = kvh % hw;
  const int t = threadIdx.x;
  const int steps = steps_of(context_lens[s]);
  const int64_t orow = row_map ? row_map[s] : s;   // wave-uniform: the block is one wave
  if (orow < 0) return;
  const int64_t row = orow * n_q + h;
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.0f;
  float inv = 0.0f;
  if (steps > 0) {
    const int64_t U = header[3];
    const int num_wgs = header[0];
    // the workgroups that ran the segment's first and last steps (the split
    // kernel records them): its pieces are theirs and those of the workgroups
    // between them; w0's piece always exists
    const int g = s * nhg + hg;
    const int w0 = seg_w[2 * g], w1 = seg_w[2 * g + 1];
    const int npc = w1 - w0 + 1;
    // Lane k holds piece w0 + b + k of a sweep over 64 pieces: first the max M
    // of the pieces' m, then each piece's weight 2^(m_k - M), broadcast while
    // every lane sums its dims of the weighted O.  A workgroup with an empty
    // unit range (only with fewer units than twice the workgroups) holds no piece; it and
    // the lanes past the last piece get weight 0 and read piece w0's O, which
    // always exists, so the O loads go out four at a time with no tail loop.
    // Most rows have at most 64 pieces: their m and l are loaded once.
    auto entry = [&](int w) -> int64_t { return (((int64_t)w + g) * hw + wv) * G + hl; };
    auto piece_ml = [&](int b, bool* has) -> float2 {
      const int w = w0 + b + t;
      // with at least twice as many units as workgroups every workgroup holds
      // a piece (a share is at least 2 * 16 / 17 units)
      *has = w <= w1 && (U >= 2 * (int64_t)num_wgs ||
                         wave_begin(w, U, num_wgs) < wave_begin(w + 1, U, num_wgs));
      return *has ? *(const float2*)(part_ml + entry(w) * 2) : make_float2(-INFINITY, 0.0f);
    };
    bool has0;
    const float2 ml0 = piece_ml(0, &has0);
    // the first four pieces' O go out with the (m, l) loads: they do not
    // depend on M, and most rows have no more pieces than that
    const uint64_t present0 = __ballot(has0);
    float o0[4][DPT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t sl = entry((present0 >> u) & 1 ? w0 + u : w0);
#pragma unroll
      for (int i = 0; i < DPT; ++i) o0[u][i] = part_o[sl * HD + t * DPT + i];
    }
    float M = ml0.x;
    for (int b = 64; b < npc; b += 64) {
      bool has;
      M = fmaxf(M, piece_ml(b, &has).x);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float lsum = 0.0f;
    for (int b = 0; b < npc; b += 64) {
      bool has = has0;
      const float2 ml = b == 0 ? ml0 : piece_ml(b, &has);
      const uint64_t present = __ballot(has);
      const float wk = has ? fast_exp2(ml.x - M) : 0.0f;
      lsum += ml.y * wk;
      const int n = min(64, npc - b);
      for (int j = 0; j < n; j += 4) {
        float o[4][DPT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t sl = entry((present >> (j + u)) & 1 ? w0 + b + j + u : w0);
#pragma unroll
          for (int i = 0; i < DPT; ++i)
            o[u][i] = b + j == 0 ? o0[u][i] : part_o[sl * HD + t * DPT + i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wj = __shfl(wk, j + u, 64);
#pragma unroll
          for (int i = 0; i < DPT; ++i) acc[i] += wj * o[u][i];
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
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
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

constexpr int MAX_WAVES_PER_CU = 32;   // upper bound used to size the workspace
constexpr int64_t MAX_WGS = 1 << 20;

// KV heads (waves) per workgroup: the largest power of two up to max_hw
// dividing n_kv.
static int heads_per_wg(int cache_dtype, int n_kv, int G) {
  int hw = max_hw(cache_dtype, G);
  while (hw > 1 && n_kv % hw) hw >>= 1;
  return hw;
}

// Number of workgroups of hw waves: the resident capacity of the device
// (auto), or one workgroup per split_tokens tokens of the largest possible
// total context (for tests).
static int64_t wgs_bound(int hw, int num_seqs, int n_kv, int max_context_len, int split_tokens) {
  if (split_tokens <= 0) return ((int64_t)device_cu_count() * MAX_WAVES_PER_CU + hw - 1) / hw;
  const int64_t units = (int64_t)num_seqs * (n_kv / hw) * units_of(max_context_len, DECODE_SEG_OV_MAX);
  const int64_t per = (split_tokens + 15) / 16;
  int64_t w = (units + per - 1) / per;
  if (w < 1) w = 1;
  if (w > MAX_WGS) w = MAX_WGS;
  return w;
}

// Partial entries (one per wave and segment piece): slots = workgroups +
// segments, hw entries per slot.  The bound covers every cache dtype, so the
// workspace size does not depend on it.
static int64_t entries_bound(int num_seqs, int n_kv, int G, int max_context_len, int split_tokens) {
  int64_t e = 0;
  for (int cdt : {(int)PA_F32, (int)PA_BF16}) {
    const int hw = heads_per_wg(cdt, n_kv, G);
    const int64_t n = (wgs_bound(hw, num_seqs, n_kv, max_context_len, split_tokens) +
                       (int64_t)num_seqs * (n_kv / hw)) * hw;
    if (n > e) e = n;
  }
  return e;
}

struct WsLayout {
  size_t hdr, seg, ml, o, total;
};
// header (256 bytes), the segments' first/last workgroups (two int32 per
// (sequence, KV head) bound), then the partials
static WsLayout ws_layout(int64_t entries, int G, int head_dim, int64_t segs) {
  WsLayout l;
  l.hdr = 0;
  l.seg = 256;
  l.ml = l.seg + align256((size_t)segs * 2 * 4);
  l.o = l.ml + align256((size_t)entries * G * 2 * 4);
  l.total = l.o + align256((size_t)entries * G * head_dim * 4);
  return l;
}

template <int CDT, int HD, int G>
static int64_t resident_wgs(int hw) {
  // per device, instantiation and group size
  static int64_t cache[MAX_DEVICES][DECODE_MAX_HW + 1] = {};
  int64_t* cached = cache[current_device()];
  if (!cached[hw]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, decode_split_kernel<CDT, HD, G, DECODE_NBUF>, 64 * hw, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    const int target = (DECODE_WAVES_PER_CU + hw - 1) / hw;
    if (per_cu > target) per_cu = target;
    cached[hw] = (int64_t)device_cu_count() * per_cu;
  }
  return cached[hw];
}

// Cache dtypes whose decode runs on the matrix cores (bit = dtype code) when
// block_size >= 16: bf16, fp8, int8 and int4.  The 8- and 4-bit codes cost
// vector-ALU work to widen, which the matrix cores take the products off (on
// the long-tail step, int4 364 -> 251 us, int8 399 -> 327 us and fp8
// 356 -> 326 us, the 8-bit caches with staged loads).  bf16 gains from the
// staged whole-row loads alone: Llama-3 GQA step 216 -> 209 us, long-tail
// step 608 -> 595 us, Llama-2 MHA unchanged at 357 us.  fp32 caches and blocks
// of fewer than 16 tokens take the vector kernel.
#ifndef DECODE_MFMA_MASK
#define DECODE_MFMA_MASK ((1 << PA_BF16) | (1 << PA_FP8_E4M3) | (1 << PA_INT8) | (1 << PA_INT4))
#endif
// steps in flight per wave on the matrix-core path.  Fewer buffers leave more
// registers to the rest of the step: on the long-tail step int4 ran at 224 us
// with two against 247-249 us with three or four, fp8 at 308 against 317 us,
// bf16 (Llama-3 and long tail) 0.2-0.4% faster; int8 312 against 308 us, so it
// keeps three (one A/B run each)
#ifndef DECODE_MF_NBUF4
#define DECODE_MF_NBUF4 2   // INT4
#endif
#ifndef DECODE_MF_NBUF8
#define DECODE_MF_NBUF8 3   // INT8
#endif
#ifndef DECODE_MF_NBUF_FP8
#define DECODE_MF_NBUF_FP8 2
#endif
#ifndef DECODE_MF_NBUF16
#define DECODE_MF_NBUF16 2   // BF16
#endif
// staged loads on the matrix-core path where the layout allows (1), or per-head
// loads everywhere (0)
#ifndef DECODE_MF_STAGED
#define DECODE_MF_STAGED 1
#endif
__host__ __device__ constexpr int mf_nbuf(int CDT) {
  return CDT == PA_INT4 ? DECODE_MF_NBUF4 : CDT == PA_BF16 ? DECODE_MF_NBUF16
       : CDT == PA_FP8_E4M3 ? DECODE_MF_NBUF_FP8 : DECODE_MF_NBUF8;
}

template <int CDT, int HD, int G, bool STAGED>
static int64_t resident_wgs_mf(int hw) {
  static int64_t cache[MAX_DEVICES][DECODE_MAX_HW + 1] = {};   // per device
  int64_t* cached = cache[current_device()];
  if (!cached[hw]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, decode_mfma_kernel<CDT, HD, G, mf_nbuf(CDT), STAGED, false>, 64 * hw, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    const int target = (DECODE_WAVES_PER_CU + hw - 1) / hw;
    if (per_cu > target) per_cu = target;
    cached[hw] = (int64_t)device_cu_count() * per_cu;
  }
  return cached[hw];
}

// The split is sized by the plain kernel in both cases, so the appending
// launch cuts the work at the same points (bit-identical results).
template <int CDT, int HD, int G, bool STAGED>
static pa_status launch_mf(const DecodeArgs& a, int split_tokens, int64_t bound, hipStream_t st) {
  DecodeArgs b = a;
  int64_t W = split_tokens <= 0 ? resident_wgs_mf<CDT, HD, G, STAGED>(a.hw) : bound;
  if (W > bound) W = bound;
  b.num_wgs = (int)W;
  if constexpr (STAGED) {
    if (a.k_new)
      return launch(decode_mfma_kernel<CDT, HD, G, mf_nbuf(CDT), STAGED, true>, dim3((unsigned)W),
                    dim3(64 * a.hw), 0, st, b);
  }
  return launch(decode_mfma_kernel<CDT, HD, G, mf_nbuf(CDT), STAGED, false>, dim3((unsigned)W),
                dim3(64 * a.hw), 0, st, b);
}

// The appending decode on paths that do not stage whole rows: the new tokens
// go to their slots in a launch of their own first.  Workgroup (s, y, K/V)
// writes 16-byte chunks of sequence s's token context_lens[s] - 1.
template <int CDT>
__global__ __launch_bounds__(256) void append_rows_kernel(DecodeArgs a, int chunks_per_row) {
  constexpr int EB = CDT == PA_F32 ? 4 : CDT == PA_BF16 ? 2 : 1;
  const int s = blockIdx.x;
  const bool is_v = blockIdx.z != 0;
  const int64_t slot = row_slot(a.block_tables + (int64_t)s * a.max_blocks, a.max_blocks,
                                a.block_size, a.bs_log2, a.context_lens[s] - 1);
  if (!is_v && blockIdx.y == 0 && threadIdx.x == 0 && a.slots_out) a.slots_out[s] = slot;
  if (slot < 0 || slot >= (int64_t)a.num_blocks * a.block_size) return;
  uint8_t* dst = (uint8_t*)(is_v ? a.v_cache : a.k_cache) + slot * a.tok_stride;
  const int64_t row0 = (int64_t)s * (a.tok_stride / EB);   // first source element of the row
  for (int c = blockIdx.y * 256 + threadIdx.x; c < chunks_per_row; c += gridDim.y * 256)
    *(uint4*)(dst + 16 * c) = new_chunk<CDT>(is_v ? a.v_new : a.k_new, row0 + 16 * c / EB,
                                              a.src_f32 != 0, is_v ? a.v_inv : a.k_inv);
}

template <int CDT>
static pa_status append_rows(DecodeArgs& a, hipStream_t st) {
  if constexpr (CDT == PA_INT4) {
    return PA_ERR_DTYPE;
  } else {
    const int chunks = (int)(a.tok_stride / 16);
    const dim3 grid((unsigned)a.num_seqs, (unsigned)((chunks + 255) / 256), 2);
    const pa_status e = launch(append_rows_kernel<CDT>, grid, dim3(256), 0, st, a, chunks);
    a.k_new = a.v_new = nullptr;   // appended: the decode reads them from the cache
    return e;
  }
}

template <int CDT, int HD, int G>
static pa_status launch_split(DecodeArgs a, int split_tokens, int max_context_len, hipStream_t st) {
  constexpr bool MF = (DECODE_MFMA_MASK >> CDT) & 1;
  const int hw = heads_per_wg(CDT, a.n_kv, G);
  const bool mf = MF && a.block_size >= 16;
  if (a.row_map && !mf) return PA_ERR_UNSUPPORTED;   // the vector kernel reads row s
  const int64_t bound = wgs_bound(hw, a.num_seqs, a.n_kv, max_context_len, split_tokens);
  a.hw = hw;
  a.nhg = a.n_kv / hw;
  if constexpr (MF) {
    if (mf) {
      if constexpr (mf_stageable_layout<CDT, HD>() && DECODE_MF_STAGED) {
        if (mf_staged_ok(MfLayout<CDT, HD>::ROW, hw))
          return launch_mf<CDT, HD, G, true>(a, split_tokens, bound, st);   // appends in the kernel
      }
      if (a.k_new) {
        const pa_status e = append_rows<CDT>(a, st);
        if (e != PA_OK) return e;
      }
      return launch_mf<CDT, HD, G, false>(a, split_tokens, bound, st);
    }
  }
  int64_t W = split_tokens <= 0 ? resident_wgs<CDT, HD, G>(hw) : bound;
  if (W > bound) W = bound;
  a.num_wgs = (int)W;
  if (a.k_new) {
    const pa_status e = append_rows<CDT>(a, st);
    if (e != PA_OK) return e;
  }
  return launch(decode_split_kernel<CDT, HD, G, DECODE_NBUF>, dim3((unsigned)W), dim3(64 * hw), 0,
                st, a);
}

template <int CDT, int HD>
static pa_status dispatch_group(int G, const DecodeArgs& a, int split_tokens, int max_ctx,
                                hipStream_t st) {
  switch (G) {
    case 1: return launch_split<CDT, HD, 1>(a, split_tokens, max_ctx, st);
    case 2: return launch_split<CDT, HD, 2>(a, split_tokens, max_ctx, st);
    case 4: return launch_split<CDT, HD, 4>(a, split_tokens, max_ctx, st);
    case 8: return launch_split<CDT, HD, 8>(a, split_tokens, max_ctx, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <int CDT>
static pa_status dispatch_hd(int hd, int G, const DecodeArgs& a, int split_tokens, int max_ctx,
                             hipStream_t st) {
  if (hd == 128) return dispatch_group<CDT, 128>(G, a, split_tokens, max_ctx, st);
  if (hd == 64) return dispatch_group<CDT, 64>(G, a, split_tokens, max_ctx, st);
  return PA_ERR_UNSUPPORTED;
}

// The merge reads the wave count the split kernel used from the workspace.
template <int HD, int G, bool BF16>
static pa_status launch_merge_t(void* out, const WsLayout& l, const void* ws, const int32_t* ctx,
                                int num_seqs, int n_kv, float out_scale, const int32_t* row_map,
                                hipStream_t st) {
  const char* base = (const char*)ws;
  return launch(decode_merge_kernel<HD, G, BF16>, dim3((unsigned)((int64_t)num_seqs * n_kv * G)),
                dim3(64), 0, st, out, (const float*)(base + l.o), (const float*)(base + l.ml),
                ctx, (const int32_t*)(base + l.hdr), (const int32_t*)(base + l.seg), num_seqs, n_kv,
                out_scale, row_map);
}

template <int HD, bool BF16>
static pa_status merge_g(int G, void* out, const WsLayout& l, const void* ws, const int32_t* ctx,
                         int num_seqs, int n_kv, float out_scale, const int32_t* row_map,
                         hipStream_t st) {
  switch (G) {
    case 1: return launch_merge_t<HD, 1, BF16>(out, l, ws, ctx, num_seqs, n_kv, out_scale, row_map, st);
    case 2: return launch_merge_t<HD, 2, BF16>(out, l, ws, ctx, num_seqs, n_kv, out_scale, row_map, st);
    case 4: return launch_merge_t<HD, 4, BF16>(out, l, ws, ctx, num_seqs, n_kv, out_scale, row_map, st);
    case 8: return launch_merge_t<HD, 8, BF16>(out, l, ws, ctx, num_seqs, n_kv, out_scale, row_map, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                            int32_t n_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t split_tokens) {
  if (num_seqs <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      n_q_heads % n_kv_heads)
    return 0;
  const int G = n_q_heads / n_kv_heads;
  return ws_layout(entries_bound(num_seqs, n_kv_heads, G, max_context_len, split_tokens), G,
                   head_dim, (int64_t)num_seqs * n_kv_heads).total;
}

static pa_status check_common(int num_seqs, int n_kv_heads, int group_size, int head_dim,
                              int max_context_len, int split_tokens) {
  if (num_seqs < 0 || n_kv_heads < 1 || group_size < 1 || max_context_len < 0 || split_tokens < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (group_size != 1 && group_size != 2 && group_size != 4 && group_size != 8)
    return PA_ERR_UNSUPPORTED;
  // units are counted in 32-bit integers
  if ((int64_t)num_seqs * n_kv_heads * units_of(max_context_len, DECODE_SEG_OV_MAX) >= (int64_t)1 << 31)
    return PA_ERR_SHAPE;
  return PA_OK;
}

static pa_status launch_merge(void* out, int out_dtype, const int32_t* context_lens, int num_seqs,
                              int n_kv, int G, int head_dim, const WsLayout& l, float out_scale,
                              const void* workspace, hipStream_t st,
                              const int32_t* row_map = nullptr) {
  if (out_dtype == PA_BF16)
    return head_dim == 128 ? merge_g<128, true>(G, out, l, workspace, context_lens, num_seqs, n_kv, out_scale, row_map, st)
                           : merge_g<64, true>(G, out, l, workspace, context_lens, num_seqs, n_kv, out_scale, row_map, st);
  return head_dim == 128 ? merge_g<128, false>(G, out, l, workspace, context_lens, num_seqs, n_kv, out_scale, row_map, st)
                         : merge_g<64, false>(G, out, l, workspace, context_lens, num_seqs, n_kv, out_scale, row_map, st);
}

// Both phases of decode; merge == false runs the partials phase only.
static pa_status decode_impl(void* out, bool merge, const void* q, int q_dtype,
                             const void* k_cache, const void* v_cache, int cache_dtype,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t head_dim, int32_t group_size, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_context_len, float scale,
                             float k_scale, float v_scale, int32_t split_tokens, void* workspace,
                             size_t workspace_bytes, void* stream,
                             const float* k_channel_scales = nullptr,
                             const float* v_token_scales = nullptr,
                             const int32_t* table_row = nullptr,
                             const void* k_new = nullptr, const void* v_new = nullptr,
                             int src_dtype = -1, int64_t* slots_out = nullptr,
                             const int32_t* row_map = nullptr) {
  pa_status e = check_common(num_seqs, n_kv_heads, group_size, head_dim, max_context_len, split_tokens);
  if (e != PA_OK) return e;
  if (num_blocks < 0 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1))) return PA_ERR_UNSUPPORTED;
  const bool int4 = cache_dtype == PA_INT4;
  const bool pair_ok = (q_dtype == PA_F32 && cache_dtype == PA_F32) ||
                       (q_dtype == PA_BF16 && (cache_dtype == PA_BF16 || cache_dtype == PA_FP8_E4M3 ||
                                                 cache_dtype == PA_INT8 || cache_dtype == PA_INT4));
  if (!pair_ok) return PA_ERR_DTYPE;
  if (num_seqs == 0) return PA_OK;
  if ((merge && !out) || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL;
  if (int4 && (!k_channel_scales || !v_token_scales)) return PA_ERR_NULL;
  const int G = group_size;
  const WsLayout l = ws_layout(
      entries_bound(num_seqs, n_kv_heads, G, max_context_len, split_tokens), G, head_dim,
      (int64_t)num_seqs * n_kv_heads);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace & 255)) return PA_ERR_WORKSPACE;
  // 8-bit caches (fp8 or int8) carry per-tensor scales
  const bool fp8 = cache_dtype == PA_FP8_E4M3 || cache_dtype == PA_INT8;
  if (fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f))) return PA_ERR_SHAPE;
  const bool append = src_dtype >= 0;
  if (append) {
    // the append's pairs: a bit copy for F32 and BF16 caches, an encode from
    // F32 or BF16 rows for FP8_E4M3 and INT8 caches (INT4: pa_kv_append_int4)
    const bool src_ok = fp8 ? (src_dtype == PA_F32 || src_dtype == PA_BF16)
                            : (!int4 && src_dtype == cache_dtype);
    if (!src_ok) return PA_ERR_DTYPE;
    if (!k_new || !v_new) return PA_ERR_NULL;
    if (((uintptr_t)k_new | (uintptr_t)v_new) & 15) return PA_ERR_SHAPE;
  }

  char* base = (char*)workspace;
  DecodeArgs a;
  a.q = (const uint8_t*)q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.header = (int32_t*)(base + l.hdr);
  a.seg_w = (int32_t*)(base + l.seg);
  a.part_ml = (float*)(base + l.ml);
  a.part_o = (float*)(base + l.o);
  const int ebits = cache_dtype == PA_F32 ? 32 : cache_dtype == PA_BF16 ? 16 : int4 ? 4 : 8;
  a.tok_stride = (int64_t)n_kv_heads * head_dim * ebits / 8;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  a.bs_log2 = lg;
  a.n_kv = n_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_wgs = 0;
  a.hw = 1;
  a.nhg = n_kv_heads;
  a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.k_ch_scale = k_channel_scales;
  a.v_tok_scale = v_token_scales;
  a.table_row = table_row;
  a.row_map = row_map;
  a.k_new = append ? (const uint8_t*)k_new : nullptr;
  a.v_new = append ? (const uint8_t*)v_new : nullptr;
  a.src_f32 = src_dtype == PA_F32;
  a.k_inv = fp8 ? 1.0f / k_scale : 1.0f;   // one binary32 division each, as pa_kv_append
  a.v_inv = fp8 ? 1.0f / v_scale : 1.0f;
  a.slots_out = append ? slots_out : nullptr;

  hipStream_t st = (hipStream_t)stream;
  if (cache_dtype == PA_BF16) e = dispatch_hd<PA_BF16>(head_dim, G, a, split_tokens, max_context_len, st);
  else if (cache_dtype == PA_FP8_E4M3) e = dispatch_hd<PA_FP8_E4M3>(head_dim, G, a, split_tokens, max_context_len, st);
  else if (cache_dtype == PA_INT8) e = dispatch_hd<PA_INT8>(head_dim, G, a, split_tokens, max_context_len, st);
  else if (int4) e = dispatch_hd<PA_INT4>(head_dim, G, a, split_tokens, max_context_len, st);
  else e = dispatch_hd<PA_F32>(head_dim, G, a, split_tokens, max_context_len, st);
  if (e != PA_OK || !merge) return e;
  return launch_merge(out, q_dtype, context_lens, num_seqs, n_kv_heads, G, head_dim, l,
                      fp8 ? v_scale : 1.0f, workspace, st, row_map);
}

extern "C" pa_status pa_decode(void* out, const void* q, int q_dtype, const void* k_cache,
                               const void* v_cache, int cache_dtype, int32_t num_blocks,
                               int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                               int32_t group_size, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t max_context_len, float scale,
                               float k_scale, float v_scale, int32_t split_tokens,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (cache_dtype == PA_INT4) return PA_ERR_DTYPE;   // its scales come through pa_decode_int4
  return decode_impl(out, true, q, q_dtype, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, n_kv_heads, head_dim, group_size, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale, k_scale,
                     v_scale, split_tokens, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_decode_partials(const void* q, int q_dtype, const void* k_cache,
                                        const void* v_cache, int cache_dtype, int32_t num_blocks,
                                        int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                                        int32_t group_size, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t max_context_len, float scale,
                                        float k_scale, int32_t split_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (cache_dtype == PA_INT4) return PA_ERR_DTYPE;   // see pa_decode_int4_partials
  return decode_impl(nullptr, false, q, q_dtype, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, n_kv_heads, head_dim, group_size, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale, k_scale,
                     1.0f, split_tokens, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_decode_append(void* out, const void* q, int q_dtype, void* k_cache,
                                      void* v_cache, int cache_dtype, int32_t num_blocks,
                                      int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t group_size, const void* k_new, const void* v_new,
                                      int src_dtype, int64_t* slot_mapping,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t max_context_len, float scale, float k_scale,
                                      float v_scale, int32_t split_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (src_dtype < 0) return PA_ERR_DTYPE;
  return decode_impl(out, true, q, q_dtype, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, n_kv_heads, head_dim, group_size, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale, k_scale,
                     v_scale, split_tokens, workspace, workspace_bytes, stream, nullptr, nullptr,
                     nullptr, k_new, v_new, src_dtype, slot_mapping);
}

extern "C" pa_status pa_decode_append_partials(const void* q, int q_dtype, void* k_cache,
                                               void* v_cache, int cache_dtype, int32_t num_blocks,
                                               int32_t block_size, int32_t n_kv_heads,
                                               int32_t head_dim, int32_t group_size,
                                               const void* k_new, const void* v_new,
                                               int src_dtype, int64_t* slot_mapping,
                                               const int32_t* block_tables,
                                               int32_t max_blocks_per_seq,
                                               const int32_t* context_lens, int32_t num_seqs,
                                               int32_t max_context_len, float scale,
                                               float k_scale, float v_scale,
                                               int32_t split_tokens, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  if (src_dtype < 0) return PA_ERR_DTYPE;
  return decode_impl(nullptr, false, q, q_dtype, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, n_kv_heads, head_dim, group_size, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale, k_scale,
                     v_scale, split_tokens, workspace, workspace_bytes, stream, nullptr, nullptr,
                     nullptr, k_new, v_new, src_dtype, slot_mapping);
}

extern "C" pa_status pa_decode_merge(void* out, int out_dtype, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t max_context_len,
                                     int32_t split_tokens, float out_scale, const void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads) return PA_ERR_SHAPE;
  const int G = n_q_heads / n_kv_heads;
  pa_status e = check_common(num_seqs, n_kv_heads, G, head_dim, max_context_len, split_tokens);
  if (e != PA_OK) return e;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !context_lens) return PA_ERR_NULL;
  const WsLayout l = ws_layout(
      entries_bound(num_seqs, n_kv_heads, G, max_context_len, split_tokens), G, head_dim,
      (int64_t)num_seqs * n_kv_heads);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace & 255)) return PA_ERR_WORKSPACE;
  return launch_merge(out, out_dtype, context_lens, num_seqs, n_kv_heads, G, head_dim, l,
                      out_scale, workspace, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// pa_decode_no_alloc: pa_decode with its split partials in a scratch array the
// library owns, for callers that cannot allocate.  The array is a file-scope
// device variable: every device the library runs on holds one copy, at its own
// address, until the process ends.  Host code must never pass the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, and is kept.
// ---------------------------------------------------------------------------
namespace pa {

static __device__ __align__(256) uint8_t scratch[PA_NO_ALLOC_SCRATCH_BYTES];

// Device address of this device's scratch copy (nullptr if it cannot be had).
static void* scratch_address() {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace pa

extern "C" pa_status pa_decode_no_alloc(void* out, const void* q, int q_dtype, const void* k_cache,
                                        const void* v_cache, int cache_dtype, int32_t num_blocks,
                                        int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                                        int32_t group_size, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t max_context_len, float scale,
                                        float k_scale, float v_scale, int32_t split_tokens,
                                        void* stream) {
  if (cache_dtype == PA_INT4) return PA_ERR_DTYPE;
  pa_status e = check_common(num_seqs, n_kv_heads, group_size, head_dim, max_context_len,
                             split_tokens);
  if (e != PA_OK) return e;
  if (num_seqs == 0) return PA_OK;
  // the partials this call needs, against the scratch's fixed size (no HIP call yet)
  const WsLayout l = ws_layout(
      entries_bound(num_seqs, n_kv_heads, group_size, max_context_len, split_tokens), group_size,
      head_dim, (int64_t)num_seqs * n_kv_heads);
  if (l.total > PA_NO_ALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return PA_ERR_HIP;
  return decode_impl(out, true, q, q_dtype, k_cache, v_cache, cache_dtype, num_blocks, block_size,
                     n_kv_heads, head_dim, group_size, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, k_scale, v_scale,
                     split_tokens, ws, PA_NO_ALLOC_SCRATCH_BYTES, stream);
}

extern "C" pa_status pa_decode_int4(void* out, const void* q, int q_dtype, const void* k_cache,
                                    const void* v_cache, const float* k_channel_scales,
                                    const float* v_token_scales, int32_t num_blocks,
                                    int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t group_size, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t max_context_len, float scale,
                                    int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return decode_impl(out, true, q, q_dtype, k_cache, v_cache, PA_INT4, num_blocks, block_size,
                     n_kv_heads, head_dim, group_size, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, 1.0f, 1.0f, split_tokens,
                     workspace, workspace_bytes, stream, k_channel_scales, v_token_scales);
}

extern "C" pa_status pa_decode_int4_partials(const void* q, int q_dtype, const void* k_cache,
                                             const void* v_cache, const float* k_channel_scales,
                                             const float* v_token_scales, int32_t num_blocks,
                                             int32_t block_size, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t group_size,
                                             const int32_t* block_tables,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t max_context_len, float scale,
                                             int32_t split_tokens, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return decode_impl(nullptr, false, q, q_dtype, k_cache, v_cache, PA_INT4, num_blocks,
                     block_size, n_kv_heads, head_dim, group_size, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, scale, 1.0f,
                     1.0f, split_tokens, workspace, workspace_bytes, stream, k_channel_scales,
                     v_token_scales);
}

// ---------------------------------------------------------------------------
// Chunked prefill over an fp32 cache (pa_prefill_chunk with F32 q and cache).
// Query row i of chunk s (L_s rows, T_s cached tokens including the chunk)
// sees the keys j <= T_s - L_s + i when causal, all T_s keys otherwise
// ("3.3 Batching and memory management", section "Chunked prefill"): that is
// a decode row of sequence s whose context is T_s - L_s + i + 1 (or T_s)
// tokens.  A planning kernel writes each row's context length and table row;
// the vector decode kernel and its merge then run over the total_q rows.
// fp32 has no matrix-core path here: every row reads its keys itself.
// ---------------------------------------------------------------------------
namespace pa {

__global__ __launch_bounds__(256) void prefill_rows_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx, int num_seqs, int total_q,
    int causal, int32_t* __restrict__ row_ctx, int32_t* __restrict__ row_seq) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= total_q) return;
  // the chunk holding row r: the last s with cu[s] <= r (cu non-decreasing)
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int c0 = cu[lo], c1 = cu[lo + 1];
  int n = 0;
  if (c0 <= r && r < c1) {
    const int T = ctx[lo];
    n = causal ? T - (c1 - c0) + (r - c0) + 1 : T;
    n = n < 0 ? 0 : n > T ? T : n;
  }
  row_ctx[r] = n;     // rows outside every chunk: no keys, zero output
  row_seq[r] = lo;
}

size_t prefill_decode_rows_workspace_bytes(int num_seqs, int n_kv, int G, int head_dim) {
  if (num_seqs <= 0) return 0;
  return ws_layout(entries_bound(num_seqs, n_kv, G, 0, 0), G, head_dim, (int64_t)num_seqs * n_kv).total;
}

pa_status prefill_decode_rows(void* out, const void* q, const void* k_cache, const void* v_cache,
                              int cache_dtype, int num_blocks, int block_size, int n_kv,
                              int head_dim, int G, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* row_ctx,
                              const int32_t* row_map, int num_seqs, int max_context_len,
                              float scale, float k_scale, float v_scale,
                              const float* k_channel_scales, const float* v_token_scales,
                              void* workspace, size_t workspace_bytes, hipStream_t st) {
  return decode_impl(out, true, q, PA_BF16, k_cache, v_cache, cache_dtype, num_blocks, block_size,
                     n_kv, head_dim, G, block_tables, max_blocks_per_seq, row_ctx, num_seqs,
                     max_context_len, scale, k_scale, v_scale, 0, workspace, workspace_bytes, st,
                     k_channel_scales, v_token_scales, nullptr, nullptr, nullptr, -1, nullptr,
                     row_map);
}

size_t prefill_f32_workspace_bytes(int total_q, int n_kv, int G, int head_dim,
                                   int max_context_len) {
  if (total_q <= 0) return 0;
  return 2 * align256((size_t)total_q * 4) +
         ws_layout(entries_bound(total_q, n_kv, G, max_context_len, 0), G, head_dim,
                   (int64_t)total_q * n_kv).total;
}

pa_status prefill_f32_rows(float* out, const float* q, const int32_t* cu_seqlens_q, int num_seqs,
                           int total_q, const void* k_cache, const void* v_cache, int num_blocks,
                           int block_size, int n_kv, int head_dim, int G,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int max_context_len, int causal,
                           float scale, void* workspace, size_t workspace_bytes,
                           hipStream_t st) {
  if ((int64_t)total_q * n_kv * units_of(max_context_len, DECODE_SEG_OV_MAX) >= (int64_t)1 << 31) return PA_ERR_SHAPE;
  const size_t rows = align256((size_t)total_q * 4);
  if (workspace_bytes < prefill_f32_workspace_bytes(total_q, n_kv, G, head_dim, max_context_len))
    return PA_ERR_WORKSPACE;
  char* base = (char*)workspace;
  int32_t* row_ctx = (int32_t*)base;
  int32_t* row_seq = (int32_t*)(base + rows);
  pa_status e = launch(prefill_rows_kernel, dim3((unsigned)((total_q + 255) / 256)), dim3(256), 0,
                       st, cu_seqlens_q, context_lens, num_seqs, total_q, causal, row_ctx,
                       row_seq);
  if (e != PA_OK) return e;
  return decode_impl(out, true, q, PA_F32, k_cache, v_cache, PA_F32, num_blocks, block_size, n_kv,
                     head_dim, G, block_tables, max_blocks_per_seq, row_ctx, total_q,
                     max_context_len, scale, 1.0f, 1.0f, 0, base + 2 * rows,
                     workspace_bytes - 2 * rows, st, nullptr, nullptr, row_seq);
}

}  // namespace pa

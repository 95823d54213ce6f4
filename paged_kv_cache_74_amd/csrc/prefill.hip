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
//     LDS, written as bf16 pairs of keys x and x + 16.  The row paddings of the K and
//     V^T buffers, with loader lanes ordered key pair first, keep the LDS
//     stores and operand reads free of bank conflicts.
//   * The scale multiplies the scores inside the exponent (one FMA).  The
//     weights are taken against the running max without looking for the
//     tile's max first; only when a lane's weights of a 16-key slice add up to
//     more than 2^PF_LOG2_TSUM does the max move (to the row's max over the
//     slice, taken on the raw scores), O get rescaled and the slice's weights get taken
//     again.  The result does not depend on which max is used.
//   * Work is balanced like the decode kernel: a unit is one 32-key tile of one
//     segment (sequence, KV head, 128-row query tile), and each resident
//     workgroup takes a contiguous range of units; segments split between
//     workgroups are combined by a log-sum-exp merge kernel.  Every segment
//     also counts a few start-up units (its query load, pipeline fill and
//     output store), and the ranges are weighted by the round in which a
//     workgroup was dispatched to its CU (see pf_wt), so that workgroups
//     finish together rather than merely holding equal tile counts.
//   * The next tile's K/V is in registers while a tile is computed; LDS is
//     double-buffered, one barrier per tile; three workgroups share a CU.
//   * Rows of length 1 (decode rows in the batch) would use one wave in four
//     and 4 of the 32 query columns of a tile.  With blocks of 16 tokens or
//     more the planner leaves them out of the tiles and lists them for the
//     decode kernel's path (decode.hip), which the call runs after the tiles.
#include "internal.h"

#include <type_traits>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#ifndef PREFILL_MIN_WGS
#define PREFILL_MIN_WGS 3   // workgroups per CU the register budget must allow
#endif

constexpr int PF_WAVES = 4;
constexpr int PF_ROWS = 32 * PF_WAVES;   // query rows per workgroup
constexpr int PF_BN = 32;                // keys per tile
constexpr int PF_LOG2_TSUM = 12;
// Start-up units per segment: a piece of a segment also loads the segment's
// queries, waits for its first tile and stores its rows (a workgroup given 28
// short causal segments took 515 us against 385 us for one given 1-2 long
// ones, at equal tile counts), and the short causal segments slow the other
// workgroups on their CU as well: with 3 start-up units the three workgroups
// on each CU holding them took 450 us against 408 us for the rest of the XCD,
// with 6 404 against 400 us, with 10 357 against 386 us.  They are units of the
// split that hold no tile.
#ifndef PF_SEG_OV
#define PF_SEG_OV 8
#endif
constexpr int PF_OV = PF_SEG_OV;
constexpr float PF_TSUM_MAX = (float)(1 << PF_LOG2_TSUM);

struct PrefillArgs {
  const uint8_t* q;          // [total_q][n_q][HD] bf16
  void* out;                 // [total_q][n_q][HD] bf16
  const int32_t* cu_q;       // [num_seqs + 1]
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* hdr;        // {segments, key tiles in all}, written by the prep kernel
  const int32_t* seg_cu;     // [segments + 1] prefix sums of key tiles per segment
  const int4* seg_desc;      // [segments] {sequence, KV head, query tile, key tiles}
  const int32_t* wg_start;   // [num_wgs][2] first (segment, unit) of each workgroup
  const int32_t* wg_begin;   // [num_wgs + 1] workgroup w takes units [wg_begin[w], wg_begin[w + 1])
  const int32_t* seg_w0;     // [segments] the workgroup holding a segment's first unit
  float* part_o;             // [slots][PF_ROWS][HD]   slot = workgroup + segment
  float* part_ml;            // [slots][PF_ROWS][2]
  int64_t tok_stride;        // bytes between consecutive tokens of a block
  int num_blocks;
  int block_size;
  int bs_log2;
  int n_kv;
  int max_blocks;
  int nseg_max;              // bound on the segments of the batch (workspace size)
  int cus;                   // compute units of the device (weights of the work split)
  int causal;
  float score_scale;         // scale * k_scale * log2(e)
  float out_scale;           // v_scale for 8-bit caches, else 1
  const float* k_ch_scale;   // INT4: [n_kv][HD] key scale per channel
  const float* v_tok_scale;  // INT4: [num_blocks][n_kv][block_size] value scale per token
};

template <int CDT, int HD>
struct PrefillLds {
  static constexpr int KROW = HD * 2 + 16;        // bytes per key row of K (padded)
  static constexpr int VROW = PF_BN * 2 + 8;      // bytes per dim row of V^T (padded)
  static constexpr int K_BYTES = PF_BN * KROW;
  static constexpr int V_BYTES = HD * VROW;
  static constexpr int SIG_BYTES = CDT == PA_INT4 ? PF_BN * 4 : 0;   // INT4 value scales
  static constexpr int BUF = K_BYTES + V_BYTES + SIG_BYTES;
};

// Tiles loaded straight into LDS (bf16 caches, head_dim 128, blocks of 16
// tokens or more): buffer loads with an LDS destination (each instruction
// writes 64 lanes x 16 bytes of LDS in lane order) fill a ring of three
// stages, two tiles ahead, with no register staging.  A stage holds the
// tile's 32 K rows and 32 V rows as they sit in the cache (256 bytes each),
// swizzled so that the operand reads meet no bank conflicts:
//   * K: 16-byte chunk c of row r at chunk c ^ (r & 15).  A score operand
//     read takes the same chunk of 16 consecutive rows per 16 lanes: 16
//     different chunk positions of the 256-byte bank window (16-byte reads
//     are served 16 lanes at a time; with c ^ (r & 7) the pattern repeated
//     every 8 rows and each read took twice its cycles).
//   * V: 64-byte block b of row r at block b ^ pfv_g(r).  The PV operand
//     (V^T, 32 dims x 16 keys) comes from two ds_read_b64_tr_b16 per MFMA:
//     each 16 lanes supply the rows of 4 keys and receive, per lane, one
//     dim's 4 values.  The 32 lanes served together read 4 rows
//     {x, x + 16, x + 1, x + 17} (x even, bit 4 clear) at one 64-byte block,
//     which pfv_g sends to 4 different blocks of a 256-byte window.
// Keys past the context load the context's last row instead (through the
// same block), so every V row in LDS is finite; their scores are masked.
constexpr int PF_DROW = 256;                    // bytes of a bf16 row at head_dim 128
constexpr int PF_DSTAGE = 2 * PF_BN * PF_DROW;  // K and V of one tile
constexpr int PF_DSTAGES = 3;
__device__ __forceinline__ int pfv_g(int r) { return (r & 1) | ((r >> 3) & 2); }
typedef short pf_s4_t __attribute__((ext_vector_type(4)));
// One buffer-to-LDS load: 16 bytes per lane at voff from r, written to LDS at
// lds_addr + 16 * lane.  Written in assembly so that the compiler, which does
// not see it, inserts no waits of its own for it: the tile loop waits for
// these loads itself (vmcnt) before the barrier that publishes a tile.  The
// instruction has no register results.
__device__ __forceinline__ void pf_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t pf_lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// Workgroups are dispatched to the chip's 8 XCDs round robin (workgroup b on
// XCD b % 8), each XCD with its own L2.  Renumbering them so that every XCD
// holds a contiguous range of the work order puts the query tiles of one
// (sequence, KV head) -- which read the same K/V tiles at about the same time
// -- on one XCD, where they share its L2 instead of each fetching from HBM.
// The renumbering is a bijection of [0, W), so correctness never depends on
// the dispatch order.
#ifndef PREFILL_XCD_LOCAL
#define PREFILL_XCD_LOCAL 1   // 0: workgroup b takes the b-th range of the work order
#endif
constexpr int PF_XCDS = 8;
__device__ __forceinline__ int xcd_local_order(int b, int W) {
  if (!PREFILL_XCD_LOCAL) return b;
  const int x = b % PF_XCDS, j = b / PF_XCDS;
  return x * (W / PF_XCDS) + min(x, W % PF_XCDS) + j;
}

// Key tiles a segment needs: up to its last query's causal limit, or all of T.
__device__ __forceinline__ int seg_tiles(int L, int T, int qt, int QB, int causal) {
  if (qt * QB >= L) return 0;
  const int last_q = min(L, (qt + 1) * QB) - 1;
  const int visible = causal ? min(T, T - L + last_q + 1) : T;
  return visible > 0 ? (visible + PF_BN - 1) / PF_BN : 0;
}

// Weights of the work split.  With R resident workgroups per CU the grid is
// dispatched in R rounds (blocks [r C, (r + 1) C) in round r), and the waves of
// the R workgroups sharing a SIMD are issued oldest first, so a workgroup of a
// later round runs slower.  A workgroup of round r takes a share of the units
// proportional to pf_wt(r).  Measured with per-workgroup timestamps on the
// mixed step (three per CU): with weights 64, 59, 50 the rounds finished at
// 316, 347 and 369 us on average; with 64, 52, 41 at 338, 337 and 350 us; with
// 64, 50, 38 at 347, 335 and 342 us (the last workgroup ended at 369, 366 and
// 362 us).  In the XCD-local work order (xcd_local_order) workgroup
// w = x M + k, M = W / 8, was block 8 k + x, of round k / (C / 8).  The weights
// only move split points; any other dispatch order gives the same results,
// only less evenly timed.
#ifndef PF_WT
#define PF_WT 64, 51, 39, 36
#endif
__device__ __forceinline__ int pf_wt(int r) {
  constexpr int t[4] = {PF_WT};
  return t[r < 4 ? r : 3];
}
// Workgroups on odd XCDs (w / (W / 8) odd in the work order) take a share
// scaled by PF_XW's second weight against the first: on the mixed step their
// workgroups took 3.1-3.7% longer at equal shares, 0.1% longer at 33 : 32.
#ifndef PF_XW
#define PF_XW 33, 32
#endif
__device__ __forceinline__ int pf_xw(int x) {
  constexpr int t[2] = {PF_XW};
  return t[x & 1];
}
// sum of the split weights of workgroups [0, w) in the work order (equal
// weights when the grid is not R whole rounds of 8-XCD-divisible CUs)
__device__ __forceinline__ int64_t pf_wsum(int w, int W, int C) {
  const bool rounds = PREFILL_XCD_LOCAL && C > 0 && C % PF_XCDS == 0 && W % C == 0 && W / C <= 4 &&
                      W % PF_XCDS == 0;
  if (!rounds) return (int64_t)w * 64;
  const int M = W / PF_XCDS, P = C / PF_XCDS, R = W / C;
  int64_t perx = 0;
  for (int r = 0; r < R; ++r) perx += (int64_t)P * pf_wt(r);
  const int q = w / M, k = w - q * M, rk = k / P;
  int64_t in = 0;   // workgroups [0, k) of XCD q
  for (int r = 0; r < rk; ++r) in += (int64_t)P * pf_wt(r);
  in += (int64_t)(k - rk * P) * pf_wt(rk);
  return ((int64_t)((q + 1) / 2) * pf_xw(0) + (int64_t)(q / 2) * pf_xw(1)) * perx + pf_xw(q) * in;
}
// first unit of workgroup w: floor(U S(w) / S(W)), S the weight prefix sum
__device__ __forceinline__ int64_t pf_split_begin(int w, int64_t U, int W, int C) {
  return U * pf_wsum(w, W, C) / pf_wsum(W, W, C);
}

// Segments of the ragged batch, in order: for each sequence s, for each KV
// head, its ceil(L_s / QB) query tiles (query tile fastest, so a workgroup
// that runs into the next segment keeps the same K/V).  A sequence with L_s = 1
// (a decode row) has one segment per KV head, a chunk of 512 queries 512 / QB
// per head: the segment count follows the batch, not num_seqs times its
// longest chunk.

// Inclusive scan of one int64 per thread over the 1024 threads of the block:
// a shuffle scan inside each wave, then one over the 16 wave totals in LDS.
// Returns the thread's inclusive prefix; *total gets the block's sum.
__device__ __forceinline__ int64_t block_scan_1024(int64_t v, int64_t* wsum, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t x = __shfl_up(v, off, 64);
    if (lane >= off) v += x;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int64_t x = __shfl_up(w, off, 64);
      if (lane >= off) w += x;
    }
    if (lane < 16) wsum[16 + lane] = w;
  }
  __syncthreads();
  const int64_t r = v + (wave > 0 ? wsum[16 + wave - 1] : 0);
  *total = wsum[31];
  __syncthreads();   // wsum is reused by the next scan
  return r;
}

// One workgroup builds the work list:
//   1. each thread counts the segments of a contiguous range of sequences; a
//      scan gives every sequence its first segment (seq_seg0, kept in LDS
//      when the batch has at most PF_PREP_LDS_SEQS sequences);
//   2. each thread takes a contiguous range of segments, writes their
//      descriptors {sequence, KV head, query tile, key tiles} and sums their
//      units (key tiles plus PF_OV start-up units for a segment with tiles);
//      a scan gives the unit prefix sums seg_cu;
//   3. the split: wg_begin[w] = pf_split_begin(w), the first unit of
//      workgroup w (kept in LDS for the searches below);
//   4. for each workgroup with units, the (segment, unit offset) holding its
//      first unit, and for each segment the workgroup holding its first unit
//      (seg_w0, read by the merge): binary searches over seg_cu and wg_begin.
// A batch whose offsets disagree with total_q and max_q_len (an offset
// outside [0, total_q], a decreasing offset or a chunk longer than max_q_len),
// which could need more segments than the workspace was sized for or reach
// rows outside q and out, or one with 2^31 key tiles or more, is given no
// work: {0, 0} in the header.
constexpr int PF_PREP_LDS_SEQS = 4095;
constexpr int PF_PREP_LDS_WGS = 2048;
constexpr int PF_PREP_LDS_SEGS = 6143;
__global__ __launch_bounds__(1024) void prefill_prep_kernel(PrefillArgs a, int num_seqs, int total_q,
                                                            int max_q_len, int QB,
                                                            int num_wgs, int32_t* __restrict__ hdr,
                                                            int32_t* __restrict__ seq_seg0_g,
                                                            int32_t* __restrict__ seg_cu,
                                                            int4* __restrict__ seg_desc,
                                                            int32_t* __restrict__ wg_start,
                                                            int32_t* __restrict__ wg_begin,
                                                            int32_t* __restrict__ seg_w0,
                                                            int32_t* __restrict__ drow_ctx,
                                                            int32_t* __restrict__ drow_map) {
  __shared__ int64_t wsum[32];
  __shared__ int32_t seq_seg0_l[PF_PREP_LDS_SEQS + 1];
  __shared__ int32_t wgb_l[PF_PREP_LDS_WGS + 1];
  __shared__ int32_t segcu_l[PF_PREP_LDS_SEGS + 1];
  const int t = threadIdx.x;
  const bool in_lds = num_seqs <= PF_PREP_LDS_SEQS;
  int32_t* seq_seg0 = in_lds ? seq_seg0_l : seq_seg0_g;
  // with drow_ctx given, rows of length 1 go to the decode path: no segments here
  auto qtiles = [&](int s) {
    const int L = max(0, a.cu_q[s + 1] - a.cu_q[s]);
    if (drow_ctx && L == 1) return 0;
    return (int)(((int64_t)L + QB - 1) / QB);
  };
  // 1. segments per sequence
  const int per_s = (num_seqs + 1023) / 1024;
  const int s0 = min(num_seqs, t * per_s), s1 = min(num_seqs, s0 + per_s);
  int64_t cs = 0;
  int bad = 0;
  for (int s = s0; s < s1; ++s) {
    const int c0 = a.cu_q[s], c1 = a.cu_q[s + 1];
    bad |= c0 < 0 || c1 < c0 || c1 > total_q || c1 - c0 > max_q_len;
    cs += (int64_t)a.n_kv * qtiles(s);
  }
  bad = __syncthreads_or(bad);
  if (drow_ctx) {   // the decode path's rows (none for a batch that breaks its bounds)
    for (int s = s0; s < s1; ++s) {
      const int c0 = a.cu_q[s];
      const bool one = !bad && a.cu_q[s + 1] - c0 == 1;
      drow_ctx[s] = one ? a.context_lens[s] : 0;
      drow_map[s] = one ? c0 : -1;
    }
  }
  int64_t nseg_all;
  const int64_t cs_end = block_scan_1024(cs, wsum, &nseg_all);
  if (bad) nseg_all = a.nseg_max + (int64_t)1;
  if (nseg_all <= a.nseg_max) {
    int64_t g = cs_end - cs;
    for (int s = s0; s < s1; ++s) {
      seq_seg0[s] = (int)g;
      g += (int64_t)a.n_kv * qtiles(s);
    }
    if (t == 1023) seq_seg0[num_seqs] = (int)g;
  }
  const int nseg = nseg_all <= a.nseg_max ? (int)nseg_all : 0;
  // the segments' unit prefix sums (and, before the scan, their tile counts)
  // in LDS for the searches of step 4 when they fit; each thread reads and
  // writes only its own segments' entries until the barrier before step 4
  const bool cu_in_lds = nseg <= PF_PREP_LDS_SEGS;
  __threadfence_block();
  __syncthreads();
  // 2. descriptors and tile counts, then their prefix sums
  const int per_g = (nseg + 1023) / 1024;
  const int g0 = min(nseg, t * per_g), g1 = min(nseg, g0 + per_g);
  int64_t ct = 0;
  if (g0 < g1) {
    int lo = 0, hi = num_seqs;               // last s with seq_seg0[s] <= g0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seq_seg0[mid] <= g0) lo = mid; else hi = mid;
    }
    int s = lo;
    for (int g = g0; g < g1; ++g) {
      while (seq_seg0[s + 1] <= g) ++s;      // skips sequences without segments
      const int L = max(0, a.cu_q[s + 1] - a.cu_q[s]);
      const int nq = qtiles(s);
      const int local = g - seq_seg0[s];
      const int kvh = local / nq, qt = local % nq;
      const int n = seg_tiles(L, a.context_lens[s], qt, QB, a.causal);
      seg_desc[g] = make_int4(s, kvh, qt, n);
      if (cu_in_lds) segcu_l[g] = n;
      ct += n > 0 ? n + PF_OV : 0;
    }
  }
  int64_t U_all;
  const int64_t ct_end = block_scan_1024(ct, wsum, &U_all);
  const bool ok = U_all < ((int64_t)1 << 31);
  const int64_t U = ok ? U_all : 0;
  const int nseg_used = ok ? nseg : 0;
  // 3. the thread's segments' prefix sums; the split
  if (ok) {
    int64_t c = ct_end - ct;
    for (int g = g0; g < g1; ++g) {
      const int n = cu_in_lds ? segcu_l[g] : seg_desc[g].w;
      seg_cu[g] = (int)c;
      if (cu_in_lds) segcu_l[g] = (int)c;
      c += n > 0 ? n + PF_OV : 0;
    }
  }
  if (t == 0) {
    seg_cu[nseg_used] = (int)U;
    if (cu_in_lds) segcu_l[nseg_used] = (int)U;
  }
  const int32_t* scu = cu_in_lds ? segcu_l : seg_cu;
  const bool wgb_in_lds = num_wgs <= PF_PREP_LDS_WGS;
  const int32_t* wgb = wgb_in_lds ? wgb_l : wg_begin;
  for (int w = t; w <= num_wgs; w += 1024) {
    const int x = (int)pf_split_begin(w, U, num_wgs, a.cus);
    wg_begin[w] = x;
    if (wgb_in_lds) wgb_l[w] = x;
  }
  __threadfence_block();
  __syncthreads();
  // 4. each workgroup's first (segment, unit): the segment whose units hold
  //    its first unit (a segment of no units is never chosen); and each
  //    segment's first workgroup, for the merge
  if (U > 0) {
    for (int w = t; w < num_wgs; w += 1024) {
      const int x = wgb[w];
      if (x >= wgb[w + 1]) continue;            // no units
      int lo = 0, hi = nseg_used;               // seg_cu[lo] <= x < seg_cu[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (scu[mid] <= x) lo = mid; else hi = mid;
      }
      wg_start[2 * w] = lo;
      wg_start[2 * w + 1] = x - scu[lo];
    }
    for (int g = g0; g < min(g1, nseg_used); ++g) {
      const int c = scu[g];
      int lo = 0, hi = num_wgs;                 // wgb[lo] <= c < wgb[hi] = U
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (wgb[mid] <= c) lo = mid; else hi = mid;
      }
      seg_w0[g] = lo;
    }
  }
  if (t == 0) {
    hdr[0] = nseg_used;
    hdr[1] = (int)U;
  }
}

// K/V element rows of one tile for this thread: keys x and x + 16 of the tile,
// chunk lc (and, for INT4, the two keys' value scales).
struct TileRegs {
  uint32_t k0[4], k1[4], v0[4], v1[4];
  float s0, s1;
};

// Pool index of token `key` clamped into [0, T): every load is issued and lands
// on a real token, so the count in flight is fixed; keys >= T are masked out
// of the scores (their probability is 0 and the clamped V row is finite).
__device__ __forceinline__ int64_t token_index(const PrefillArgs& a, const int32_t* table, int key,
                                               int T) {
  const int kc = min(key, T - 1);
  const int j = min(kc >> a.bs_log2, a.max_blocks - 1);
  int blk = table[j];
  blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
  return (int64_t)blk * a.block_size + (kc & (a.block_size - 1));
}

template <int CDT>
__device__ __forceinline__ void load8(const uint8_t* p, uint32_t (&d)[4]) {
  if constexpr (CDT == PA_BF16) {
    const uint4 x = *(const uint4*)p;
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
  } else if constexpr (CDT == PA_INT4) {   // 8 codes in 4 bytes, widened when stored
    d[0] = *(const uint32_t*)p; d[1] = 0u; d[2] = 0u; d[3] = 0u;
  } else {   // 8-bit codes: keep the raw bytes, widened when stored to LDS
    const uint2 x = *(const uint2*)p;
    d[0] = x.x; d[1] = x.y; d[2] = 0u; d[3] = 0u;
  }
}

// The same through a buffer descriptor: a wave-uniform base in scalar
// registers plus a 32-bit lane offset, so no 64-bit lane address is built.
typedef uint32_t pf_u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t pf_u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  // 4th descriptor word for the gfx9 family: 32-bit data format, raw addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <int CDT>
__device__ __forceinline__ void load8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&d)[4]) {
  if constexpr (CDT == PA_BF16) {
    const pf_u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
  } else if constexpr (CDT == PA_INT4) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); d[1] = 0u; d[2] = 0u; d[3] = 0u;
  } else {
    const pf_u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    d[0] = x.x; d[1] = x.y; d[2] = 0u; d[3] = 0u;
  }
}

// 8 codes -> 4 bf16 pairs (exact).  INT4 pairs come out as elements (0,2)
// (4,6) (1,3) (5,7) of the 8 (the converter's order); the others in order.
template <int CDT>
__device__ __forceinline__ void widen(uint32_t (&d)[4]) {
  if constexpr (CDT == PA_FP8_E4M3 || CDT == PA_INT8) {
    const uint32_t x = d[0], y = d[1];
    d[0] = code8x2_to_bf16x2<CDT, false>(x); d[1] = code8x2_to_bf16x2<CDT, true>(x);
    d[2] = code8x2_to_bf16x2<CDT, false>(y); d[3] = code8x2_to_bf16x2<CDT, true>(y);
  } else if constexpr (CDT == PA_INT4) {
    const uint32_t lo = int4_lo_as_e4m3(d[0]), hi = int4_hi_as_e4m3(d[0]);
    d[0] = int4e4m3_to_bf16x2<false>(lo); d[1] = int4e4m3_to_bf16x2<true>(lo);
    d[2] = int4e4m3_to_bf16x2<false>(hi); d[3] = int4e4m3_to_bf16x2<true>(hi);
  }
}
// element of the 8 that pair i of widen() holds in its low (HI = false) or high half
template <int CDT>
__device__ __forceinline__ int widened_elem(int i, bool hi) {
  if constexpr (CDT == PA_INT4) return (i & 1) * 4 + (i >> 1) + (hi ? 2 : 0);
  else return 2 * i + (hi ? 1 : 0);
}

template <int CDT, int HD, int G, bool DIRECT>
__device__ __forceinline__ void prefill_piece(const PrefillArgs& a, int g, int t0, int t1, int nt,
                                              int split, int wg, uint8_t* lds) {
  static_assert(!DIRECT || (CDT == PA_BF16 && HD == 128), "direct tiles: bf16, head_dim 128");
  using LD = PrefillLds<CDT, HD>;
  constexpr int QB = PF_ROWS / G;            // queries per segment
  constexpr int EBITS = CDT == PA_BF16 ? 16 : CDT == PA_INT4 ? 4 : 8;
  constexpr int ROWB = HD * EBITS / 8;       // bytes of one (token, head) row in the cache
  constexpr int NDT = HD / 32;               // 32-dim output tiles
  constexpr int NKT = HD / 16;               // 16-dim steps of the score MFMA
  constexpr int CHUNKS = HD / 8;
  constexpr int BUF = LD::BUF;

  const int32_t* desc = (const int32_t*)a.seg_desc + 4 * (int64_t)g;
  const int s = uniform_load(desc, 0), kvh = uniform_load(desc, 1), qt = uniform_load(desc, 2);
  const int q0 = a.cu_q[s];
  const int L = a.cu_q[s + 1] - q0;
  const int T = a.context_lens[s];
  const int n_q = a.n_kv * G;

  // Rows are query-major: row rr is query qt * QB + rr / G of head rr % G, so
  // the valid rows of a short segment (a decode row has G of them) fill the
  // first wave, and a wave whose queries all lie past the end of the chunk
  // only helps stage the K/V tiles.
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, grp = lane >> 5;
  const int rr = wave * 32 + lr;             // row of the segment
  const int hl = rr % G;
  const int qi = qt * QB + rr / G;
  const bool row_ok = qi < L;
  const bool wave_ok = qt * QB + wave * 32 / G < L;
  const int pos = T - L + qi;
  const int head = kvh * G + hl;

  uint32_t qreg[NKT][4];
  {
    const int qrow = row_ok ? qi : 0;
    const uint8_t* qp = a.q + ((int64_t)(q0 + qrow) * n_q + head) * HD * 2 + grp * 16;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const uint4 x = *(const uint4*)(qp + t * 32);
      qreg[t][0] = x.x; qreg[t][1] = x.y; qreg[t][2] = x.z; qreg[t][3] = x.w;
      if constexpr (CDT == PA_INT4) {
        // times each channel's key scale, rounded to bf16, in the order the
        // widened key codes sit in LDS
        const float* ks = a.k_ch_scale + (int64_t)kvh * HD + 16 * t + 8 * grp;
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16lo_f32(w[e]) * ks[2 * e];
          f[2 * e + 1] = bf16hi_f32(w[e]) * ks[2 * e + 1];
        }
        qreg[t][0] = pack_bf16(f[0], f[2]); qreg[t][1] = pack_bf16(f[4], f[6]);
        qreg[t][2] = pack_bf16(f[1], f[3]); qreg[t][3] = pack_bf16(f[5], f[7]);
      }
    }
  }
  const int first_pos = T - L + qt * QB;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;

  f32x16_t acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
  float m = -1e30f, lsum = 0.0f;
  const float c = a.score_scale;

  // thread -> (key pair, 8-element chunk), key pair fastest.  Pair x holds
  // keys x and x + 16 of the tile: with blocks of 16 tokens the two keys lie
  // in the two blocks the tile spans, at the same offset, so each load
  // instruction reads one block (a scalar base plus a 32-bit lane offset that
  // does not change from tile to tile).  V^T stores pair x as one bf16 pair at
  // byte 4x of a dim row; the 16 lanes that share a chunk write 16 different
  // pairs of the same rows, which with the row paddings above keeps every LDS
  // store and operand read free of bank conflicts.  With head_dim 64 the upper
  // half of the workgroup repeats the lower half's loads and (identical) LDS
  // stores, so no branch separates loading threads and the wait counts stay
  // exact
  const int lp = tid % (PF_BN / 2);
  const int lc = (tid / (PF_BN / 2)) % CHUNKS;
  constexpr bool loader = true;
  const int64_t col = (int64_t)kvh * ROWB + lc * EBITS;   // 8 elements of EBITS bits
  // blocks of 16 tokens or more: byte offset of key x inside its block's rows
  const uint32_t lane_off = (uint32_t)(lp * a.tok_stride + col);
  const int64_t blk_bytes = (int64_t)a.block_size * a.tok_stride;

  const int jmax = min((T - 1) >> a.bs_log2, a.max_blocks - 1);
  // table entries of tile t (blocks of 16 tokens or more): read a tile ahead of
  // the tile's loads, so their scalar loads return while a tile is computed
  auto tab = [&](int t, int& b0, int& b1) {
    if (a.block_size >= 16) {
      const int jlo = min((t * PF_BN) >> a.bs_log2, jmax);
      b0 = uniform_load(table, jlo);
      b1 = uniform_load(table, min(jlo + 1, jmax));
    }
  };
  auto gload = [&](int t, int blo, int b1, TileRegs& R) {
    if (a.block_size >= 16) {
      b1 = a.block_size != 16 ? blo : b1;
      const int inb = (t * PF_BN) & (a.block_size - 1);   // first key's offset in its block
      const int inb1 = a.block_size == 16 ? 0 : inb + 16;
      const int64_t off0 = blo * blk_bytes + inb * a.tok_stride;
      const int64_t off1 = b1 * blk_bytes + inb1 * a.tok_stride;
      const int32_t nb0 = (int32_t)(blk_bytes - inb * a.tok_stride);
      const int32_t nb1 = (int32_t)(blk_bytes - inb1 * a.tok_stride);
      load8_buf<CDT>(make_rsrc(a.k_cache + off0, nb0), lane_off, R.k0);
      load8_buf<CDT>(make_rsrc(a.k_cache + off1, nb1), lane_off, R.k1);
      load8_buf<CDT>(make_rsrc(a.v_cache + off0, nb0), lane_off, R.v0);
      load8_buf<CDT>(make_rsrc(a.v_cache + off1, nb1), lane_off, R.v1);
      if constexpr (CDT == PA_INT4) {   // the two keys' value scales ([block][head][offset])
        const float* vs = a.v_tok_scale + (int64_t)kvh * a.block_size + lp;
        const int64_t hb = (int64_t)a.n_kv * a.block_size;
        R.s0 = vs[blo * hb + inb];
        R.s1 = vs[b1 * hb + inb1];
      }
    } else {
      // smaller blocks: each key through its own table entry, clamped into
      // the context, so every load lands on a real token
      const int64_t tk0 = token_index(a, table, t * PF_BN + lp, T);
      const int64_t tk1 = token_index(a, table, t * PF_BN + lp + 16, T);
      const int64_t o0 = tk0 * a.tok_stride + col, o1 = tk1 * a.tok_stride + col;
      load8<CDT>(a.k_cache + o0, R.k0);
      load8<CDT>(a.k_cache + o1, R.k1);
      load8<CDT>(a.v_cache + o0, R.v0);
      load8<CDT>(a.v_cache + o1, R.v1);
      if constexpr (CDT == PA_INT4) {
        R.s0 = a.v_tok_scale[((tk0 >> a.bs_log2) * a.n_kv + kvh) * a.block_size + (tk0 & (a.block_size - 1))];
        R.s1 = a.v_tok_scale[((tk1 >> a.bs_log2) * a.n_kv + kvh) * a.block_size + (tk1 & (a.block_size - 1))];
      }
    }
  };
  auto sstore = [&](TileRegs& R, uint8_t* buf, int t) {
    if (loader) {
      widen<CDT>(R.k0); widen<CDT>(R.k1); widen<CDT>(R.v0); widen<CDT>(R.v1);
      if (t * PF_BN + PF_BN > T) {
        // the context ends inside this tile: keys past it hold stale rows,
        // whose weight is 0; their V (and INT4 value scale) must be finite
        const bool z0 = t * PF_BN + lp >= T, z1 = t * PF_BN + lp + 16 >= T;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          R.v0[i] = z0 ? 0u : R.v0[i];
          R.v1[i] = z1 ? 0u : R.v1[i];
        }
        if constexpr (CDT == PA_INT4) {
          R.s0 = z0 ? 0.0f : R.s0;
          R.s1 = z1 ? 0.0f : R.s1;
        }
      }
      uint8_t* lk = buf;
      uint8_t* lv = buf + LD::K_BYTES;
      *(uint4*)(lk + lp * LD::KROW + lc * 16) = make_uint4(R.k0[0], R.k0[1], R.k0[2], R.k0[3]);
      *(uint4*)(lk + (lp + 16) * LD::KROW + lc * 16) = make_uint4(R.k1[0], R.k1[1], R.k1[2], R.k1[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // V^T[d][x, x + 16] as bf16 pairs
        const int dl = lc * 8 + widened_elem<CDT>(i, false);
        const int dh = lc * 8 + widened_elem<CDT>(i, true);
        *(uint32_t*)(lv + dl * LD::VROW + 4 * lp) = pair_lo(R.v0[i], R.v1[i]);
        *(uint32_t*)(lv + dh * LD::VROW + 4 * lp) = pair_hi(R.v0[i], R.v1[i]);
      }
      // INT4 value scales in pair order: (sigma[x], sigma[x + 16]) at byte 8x
      if constexpr (CDT == PA_INT4)
        if (lc == 0) *(float2*)(buf + LD::K_BYTES + LD::V_BYTES + 8 * lp) = make_float2(R.s0, R.s1);
    }
  };
  // MASKED is a compile-time flag: only the last tiles of a segment hold keys
  // that some row must not see, and the others skip the mask's compares and
  // selects entirely
  auto compute = [&](const uint8_t* buf, int kt, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint8_t* lk = buf;
    const uint8_t* lv = buf + (DIRECT ? PF_BN * PF_DROW : LD::K_BYTES);
    const int kb = kt * PF_BN;
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const uint4 kx = DIRECT ? *(const uint4*)(lk + lr * PF_DROW + 16 * ((2 * t + grp) ^ (lr & 15)))
                              : *(const uint4*)(lk + lr * LD::KROW + (16 * t + 8 * grp) * 2);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, kx);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(qreg[t][0], qreg[t][1], qreg[t][2], qreg[t][3]));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, sc, 0, 0, 0);
    }
    // raw scores; the positive scale c is applied inside the exponent below
    if constexpr (MASKED) {
      // score r holds key kb + 4 grp + 8(r/4) + r%4; keys above the row's last
      // visible key are masked
      const int lim = (a.causal ? min(pos, T - 1) : T - 1) - kb - 4 * grp;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) <= lim ? sc[r] : -INFINITY;
    }
    // INT4: the value scales of this lane's keys in pair order: sg[8 s + 2 i]
    // and sg[8 s + 2 i + 1] belong to keys 8 s + 4 grp + i and that + 16
    float sg[16];
    if constexpr (CDT == PA_INT4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x = *(const float4*)(buf + LD::K_BYTES + LD::V_BYTES + 32 * grp + 64 * (q >> 1) + 16 * (q & 1));
        sg[4 * q] = x.x; sg[4 * q + 1] = x.y; sg[4 * q + 2] = x.z; sg[4 * q + 3] = x.w;
      }
    }
    // O^T += V^T P^T over two 16-key slices.  Score r of this lane is key
    // 4 grp + 8 (r / 4) + r % 4; slice s pairs score r = 4 s + i with r + 8
    // (keys x and x + 16, x = 8 s + 4 grp + i), the pair order of V^T in LDS.
    //
    // The weights are taken against the running max m without first finding
    // the tile's max.  m moves only when the weights of a slice of some lane
    // add up to more than 2^PF_LOG2_TSUM (always so on a segment's first tile,
    // where m starts far below every score): then it moves to the row's max
    // over the slice, O and l are rescaled and the slice's weights taken
    // again.  Otherwise every weight 2^(s c - m) is at most 2^PF_LOG2_TSUM,
    // so O and l stay far from overflow, and O / l does not depend on which
    // m was used.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t P[4];
      float ts;
      auto weights = [&]() {
        ts = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(sc[4 * s + i], c, -m));
          const float p1 = fast_exp2(__builtin_fmaf(sc[4 * s + i + 8], c, -m));
          if constexpr (CDT == PA_INT4) {   // value scale into the weight; l unscaled, fp32
            P[i] = pack_bf16(p0 * sg[8 * s + 2 * i], p1 * sg[8 * s + 2 * i + 1]);
            ts += p0 + p1;
          } else {
            P[i] = pack_bf16(p0, p1);
            ts = dot2_bf16(P[i], 0x3F803F80u, ts);
          }
        }
      };
      weights();
      if (__any(!(ts <= PF_TSUM_MAX))) {
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, fmaxf(sc[4 * s + i], sc[4 * s + i + 8]));
        tmax = fmaxf(tmax, shfl_xor(tmax, 32));
        const float mn = fmaxf(m, tmax * c);
        const float alpha = fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
        m = mn;
        weights();
      }
      lsum += ts;
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(P[0], P[1], P[2], P[3]));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {   // V^T pairs x = 8 s + 4 grp .. + 3 of dim row 32 dt + lr
        bf16x8_t av;
        if constexpr (DIRECT) {
          // lane 16 j + i: key rows x + {0, 16, 1, 17}[i / 4] (+ 2 in the second read),
          // x = 8 s + 4 grp, bytes 32 (j % 2) + 8 (i % 4) of 64-byte block dt; it
          // receives dim 32 dt + 16 (j % 2) + i of those rows, the keys in the
          // pair order of the weights: x, x + 16, x + 1, x + 17, x + 2, ...
          const int i4 = (lane & 15) >> 2;
          const int r1 = 8 * s + 4 * grp + (i4 >> 1) + 16 * (i4 & 1), r2 = r1 + 2;
          const int cb = 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
          const pf_s4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) pf_s4_t*)(lv + r1 * PF_DROW + 64 * (dt ^ pfv_g(r1)) + cb));
          const pf_s4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) pf_s4_t*)(lv + r2 * PF_DROW + 64 * (dt ^ pfv_g(r2)) + cb));
          const uint2 lo = __builtin_bit_cast(uint2, v1), hi = __builtin_bit_cast(uint2, v2);
          av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          const uint8_t* vrow = lv + (32 * dt + lr) * LD::VROW + 32 * s + 16 * grp;
          const uint2 lo = *(const uint2*)vrow;
          const uint2 hi = *(const uint2*)(vrow + 8);
          av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[dt], 0, 0, 0);
      }
    }
  };

  // tiles below tfull hold only keys that every row of the segment sees
  const int tfull = min(T, a.causal ? first_pos + 1 : T) / PF_BN;
  // Order of the key tiles: step i < tfull computes tile (i + rot) mod tfull,
  // the masked tiles follow in order.  rot makes the piece that starts at the
  // segment's first split point (step `split`) start at tile 0, so that the
  // workgroups starting at the k-th split point of the query tiles of one
  // (sequence, KV head) read the same K/V tiles at about the same time and
  // share them in L2.  Any order gives the same (m, l, O) up to rounding; the
  // order is fixed by the plan, so results do not change from run to run.
  const int rot = tfull > 0 ? (tfull - split % tfull) % tfull : 0;
  auto tile_of = [&](int i) { return i < tfull ? (i + rot < tfull ? i + rot : i + rot - tfull) : i; };
  if constexpr (!DIRECT) {
  // the next tile in registers while one is computed, two LDS buffers.  One
  // loop body per tile (the buffer offset alternates at run time) keeps the
  // accumulators in the same registers from tile to tile.
  TileRegs R0;
  int nb0 = 0, nb1 = 0;
  tab(tile_of(t0), nb0, nb1);
  nb0 = (unsigned)nb0 < (unsigned)a.num_blocks ? nb0 : 0;
  nb1 = (unsigned)nb1 < (unsigned)a.num_blocks ? nb1 : 0;
  gload(tile_of(t0), nb0, nb1, R0);
  tab(tile_of(min(t0 + 1, t1 - 1)), nb0, nb1);
  nb0 = (unsigned)nb0 < (unsigned)a.num_blocks ? nb0 : 0;
  nb1 = (unsigned)nb1 < (unsigned)a.num_blocks ? nb1 : 0;
  int boff = 0;
  auto tile = [&](int t, auto masked) {
    sstore(R0, lds + boff, tile_of(t));
    gload(tile_of(min(t + 1, t1 - 1)), nb0, nb1, R0);
    __syncthreads();
    tab(tile_of(min(t + 2, t1 - 1)), nb0, nb1);
    if (wave_ok) compute(lds + boff, tile_of(t), masked);
    // ids outside the pool read block 0 (their keys are past the context or
    // the table breaks its contract); checked here, after the tile, where the
    // scalar loads have long returned
    nb0 = (unsigned)nb0 < (unsigned)a.num_blocks ? nb0 : 0;
    nb1 = (unsigned)nb1 < (unsigned)a.num_blocks ? nb1 : 0;
    boff ^= BUF;
  };
  const int tm = max(t0, min(t1, tfull));
  for (int t = t0; t < tm; ++t) tile(t, std::false_type{});
  for (int t = tm; t < t1; ++t) tile(t, std::true_type{});
  } else {
    // Wave w loads K and V rows 8 w .. 8 w + 7 of a tile, two buffer-to-LDS
    // instructions each (rows 8 w + 4 n .. + 3): lane i takes row
    // 8 w + 4 n + i / 16 and the 16 bytes for LDS chunk i % 16.  Waves 0-1
    // read the block of the tile's first key, waves 2-3 that of key 16 (the
    // next table entry with blocks of 16 tokens, the same block otherwise).
    const int prow = 8 * wave + (lane >> 4), pch = lane & 15;
    const int64_t blk_bytes = (int64_t)a.block_size * a.tok_stride;
    auto issue = [&](int t, int stage) {
      const int jlo = min((t * PF_BN) >> a.bs_log2, jmax);
      const int j = (wave >= 2 && a.block_size == 16) ? min(jlo + 1, jmax) : jlo;
      int blk = uniform_load(table, j);
      blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
      const int kstart = j << a.bs_log2;   // key of the block's first row
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_cache + blk * blk_bytes, (int32_t)blk_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_cache + blk * blk_bytes, (int32_t)blk_bytes);
      uint8_t* st = lds + stage * PF_DSTAGE;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int R = prow + 4 * n;
        const int key = min(t * PF_BN + R, T - 1);   // past the context: its last row
        const uint32_t ro = (uint32_t)((int64_t)(key - kstart) * a.tok_stride + kvh * PF_DROW);
        const uint32_t ko = ro + 16 * (pch ^ (R & 15));
        const uint32_t vo = ro + 16 * (4 * ((pch >> 2) ^ pfv_g(R)) + (pch & 3));
        const int rowb = (8 * wave + 4 * n) * PF_DROW;
        pf_load_lds16(rk, ko, __builtin_amdgcn_readfirstlane(pf_lds_addr(st + rowb)));
        pf_load_lds16(rv, vo, __builtin_amdgcn_readfirstlane(pf_lds_addr(st + PF_BN * PF_DROW + rowb)));
      }
    };
    // two tiles ahead; before a tile is read, this wave's four loads of it
    // have landed (at most the four of the next tile still in flight), and
    // the barrier makes every wave's visible and frees the stage the tile two
    // ahead then goes to.  The first tile's loads and the query fragments are
    // waited for together before the second tile is issued, so that no load
    // the compiler tracks is still in flight in the loop (it would otherwise
    // wait for all loads, the tile two ahead's among them, before the MFMAs)
    issue(tile_of(t0), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (t0 + 1 < t1) issue(tile_of(t0 + 1), 1);
    int stage = 0;
    auto dtile = [&](int t, auto masked) {
      if (t + 1 < t1) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
      else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (t + 2 < t1) issue(tile_of(t + 2), stage == 0 ? 2 : stage - 1);
      if (wave_ok) compute(lds + stage * PF_DSTAGE, tile_of(t), masked);
      stage = stage == 2 ? 0 : stage + 1;
    };
    const int tm = max(t0, min(t1, tfull));
    for (int t = t0; t < tm; ++t) dtile(t, std::false_type{});
    for (int t = tm; t < t1; ++t) dtile(t, std::true_type{});
  }
  __syncthreads();   // the next piece reuses the LDS buffers

  const float ltot = lsum + shfl_xor(lsum, 32);
  if (t0 == 0 && t1 == nt) {
    // the whole segment: normalise and store the output rows
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
  } else {
    // a piece: unnormalised (m, l, O) of every row into slot wg + g
    const int64_t slot = (int64_t)wg + g;
    float* po = a.part_o + (slot * PF_ROWS + rr) * HD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * grp;
        *(float4*)(po + d) = make_float4(acc[dt][4 * r4 + 0], acc[dt][4 * r4 + 1],
                                         acc[dt][4 * r4 + 2], acc[dt][4 * r4 + 3]);
      }
    if (grp == 0) *(float2*)(a.part_ml + (slot * PF_ROWS + rr) * 2) = make_float2(m, ltot);
  }
}

template <int CDT, int HD, int G, bool DIRECT>
__global__ __launch_bounds__(256, PREFILL_MIN_WGS) void prefill_kernel(PrefillArgs a) {
  using LD = PrefillLds<CDT, HD>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[DIRECT ? PF_DSTAGES * PF_DSTAGE : 2 * LD::BUF];
  const int W = gridDim.x;
  const int wg = xcd_local_order(blockIdx.x, W);
  const int64_t u0 = uniform_load(a.wg_begin, wg), u1 = uniform_load(a.wg_begin, wg + 1);
  if (u0 >= u1) return;
  int g = a.wg_start[2 * wg];
  int off = a.wg_start[2 * wg + 1];
  int64_t u = u0;
  // segment g holds units [seg_cu[g], seg_cu[g + 1]): PF_OV start-up units,
  // then its key tiles; a range that holds only start-up units of a segment
  // computes nothing there
  while (true) {
    const int c0 = uniform_load(a.seg_cu, g);
    const int nu = uniform_load(a.seg_cu, g + 1) - c0;
    const int end = (int)min((int64_t)nu, off + (u1 - u));
    const int tb = max(off - PF_OV, 0), te = max(end - PF_OV, 0);
    if (te > tb) {
      // the segment's first split point: where the workgroup after the one
      // holding its first unit begins (past the segment if none does)
      const int split = max(uniform_load(a.wg_begin, uniform_load(a.seg_w0, g) + 1) - c0 - PF_OV, 0);
      prefill_piece<CDT, HD, G, DIRECT>(a, g, tb, te, nu - PF_OV, split, wg, lds);
    }
    u += end - off;
    if (u >= u1) break;
    do { ++g; } while (uniform_load(a.seg_cu, g + 1) == uniform_load(a.seg_cu, g));
    off = 0;
  }
}

// Combine the pieces of segments split between workgroups (segments done by
// one workgroup were written directly).  The workgroups holding a segment's
// units are seg_w0[g], seg_w0[g] + 1, ... up to the one whose range passes the
// segment's end; each contributes the key tiles of its range (a range inside
// the start-up units contributes none).  Workgroup (g, part) takes NP passes
// of 256 / (HD / 4) rows of segment g; each row is read by HD / 4 consecutive
// lanes (four dims each), so every load and store of a wave covers whole rows,
// and each thread merges NP row slices in one online pass over the pieces,
// their loads of a piece issued together.  On the mixed step (HD 128) the
// merge took 18.8 us with one pass of 8 rows, 16.9 us with two (16 rows),
// 16.9-17.4 us with four and 18.2-18.5 us with eight.
template <int HD>
struct MergeShape {
  static constexpr int LPR = HD / 4;            // lanes per row
  static constexpr int RPP = 256 / LPR;         // rows per pass of the workgroup
  static constexpr int NP = 2;                  // passes per workgroup
  static constexpr int ROWS = RPP * NP;         // rows per workgroup
};
template <int HD, int G>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a, int num_wgs) {
  constexpr int QB = PF_ROWS / G;
  constexpr int LPR = MergeShape<HD>::LPR;
  constexpr int RPP = MergeShape<HD>::RPP;
  constexpr int NP = MergeShape<HD>::NP;
  constexpr int ROWS = MergeShape<HD>::ROWS;
  static_assert(PF_ROWS % ROWS == 0, "merge tiling");
  const int g = blockIdx.x / (PF_ROWS / ROWS);
  const int part = blockIdx.x % (PF_ROWS / ROWS);
  if (g >= a.hdr[0]) return;
  const int64_t c0 = a.seg_cu[g], c1 = a.seg_cu[g + 1];
  if (c1 <= c0) return;
  const int w0 = a.seg_w0[g];
  if (a.wg_begin[w0 + 1] >= c1) return;          // one workgroup wrote the whole segment
  const int4 dsc = a.seg_desc[g];
  const int s = dsc.x, kvh = dsc.y, qt = dsc.z;
  const int q0 = a.cu_q[s];
  const int L = a.cu_q[s + 1] - q0;
  const int n_q = a.n_kv * G;
  const int d0 = (threadIdx.x % LPR) * 4;
  const int r0 = part * ROWS + threadIdx.x / LPR;
  float4 acc[NP];
  float M[NP], lsum[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) { acc[p] = make_float4(0.0f, 0.0f, 0.0f, 0.0f); M[p] = -INFINITY; lsum[p] = 0.0f; }
  const int nt = (int)(c1 - c0) - PF_OV;
  for (int w = w0; w < num_wgs; ++w) {
    const int64_t wb = a.wg_begin[w], we = a.wg_begin[w + 1];
    if (wb >= c1) break;
    const int64_t b = max(wb, c0) - c0, e = min(we, c1) - c0;
    const int64_t tb = max(b - PF_OV, (int64_t)0), te = max(e - PF_OV, (int64_t)0);
    if (te <= tb) continue;                       // no tile of this segment
    if (tb == 0 && te == nt) return;              // the whole segment, written directly
    const int64_t base = ((int64_t)w + g) * PF_ROWS + r0;
    float2 ml[NP];
    float4 o[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t row = base + p * RPP;
      ml[p] = *(const float2*)(a.part_ml + row * 2);
      o[p] = *(const float4*)(a.part_o + row * HD + d0);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float Mn = fmaxf(M[p], ml[p].x);
      const float x = fast_exp2(M[p] - Mn), y = fast_exp2(ml[p].x - Mn);
      lsum[p] = lsum[p] * x + ml[p].y * y;
      acc[p].x = acc[p].x * x + o[p].x * y; acc[p].y = acc[p].y * x + o[p].y * y;
      acc[p].z = acc[p].z * x + o[p].z * y; acc[p].w = acc[p].w * x + o[p].w * y;
      M[p] = Mn;
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int rr = r0 + p * RPP;
    const int qi = qt * QB + rr / G;
    if (qi >= L) continue;
    const float inv = lsum[p] > 0.0f ? a.out_scale / lsum[p] : 0.0f;
    uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + qi) * n_q + kvh * G + rr % G) * HD + d0;
    *(uint2*)orow = make_uint2(pack_bf16(acc[p].x * inv, acc[p].y * inv),
                               pack_bf16(acc[p].z * inv, acc[p].w * inv));
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t pf_align(size_t x) { return (x + 255) & ~(size_t)255; }

static int pf_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

constexpr int PF_MAX_WGS_PER_CU = 4;   // bounds the workspace (LDS allows at most 4)

// The workspace: the plan and partials of the tile kernel, then the rows of
// length 1 for the decode path (their contexts and q/out rows, and the decode
// split's partials).
struct PfLayout {
  size_t hdr, seq, seg, desc, wgs, wgb, sw0, ml, o, drow_ctx, drow_map, dws, dws_bytes, total;
};
static PfLayout pf_layout(int64_t num_seqs, int64_t nseg, int64_t wgs, int head_dim, int n_kv,
                          int G) {
  PfLayout l;
  const size_t slots = (size_t)(wgs + nseg);
  l.hdr = 0;
  l.seq = 256;
  l.seg = l.seq + pf_align((size_t)(num_seqs + 1) * 4);
  l.desc = l.seg + pf_align((size_t)(nseg + 1) * 4);
  l.wgs = l.desc + pf_align((size_t)nseg * 16);
  l.wgb = l.wgs + pf_align((size_t)wgs * 2 * 4);
  l.sw0 = l.wgb + pf_align((size_t)(wgs + 1) * 4);
  l.ml = l.sw0 + pf_align((size_t)nseg * 4);
  l.o = l.ml + pf_align(slots * PF_ROWS * 2 * 4);
  l.drow_ctx = l.o + pf_align(slots * PF_ROWS * head_dim * 4);
  l.drow_map = l.drow_ctx + pf_align((size_t)num_seqs * 4);
  l.dws = l.drow_map + pf_align((size_t)num_seqs * 4);
  l.dws_bytes = prefill_decode_rows_workspace_bytes((int)num_seqs, n_kv, G, head_dim);
  l.total = l.dws + pf_align(l.dws_bytes);
  return l;
}

template <int CDT, int HD, int G, bool DIRECT>
static int pf_resident_wgs() {
  static int cache[MAX_DEVICES] = {};   // per device and instantiation
  int& cached = cache[current_device()];
  if (!cached) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<CDT, HD, G, DIRECT>, 256, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
    if (per_cu > PF_MAX_WGS_PER_CU) per_cu = PF_MAX_WGS_PER_CU;
    cached = pf_cu_count() * per_cu;
  }
  return cached;
}

template <int CDT, int HD, int G, bool DIRECT>
static pa_status pf_launch_k(PrefillArgs a, int num_seqs, int total_q, int max_q_len,
                             const PfLayout& l, char* ws, bool route, hipStream_t st) {
  const int W = pf_resident_wgs<CDT, HD, G, DIRECT>();
  a.hdr = (const int32_t*)(ws + l.hdr);
  a.seg_cu = (const int32_t*)(ws + l.seg);
  a.seg_desc = (const int4*)(ws + l.desc);
  a.wg_start = (const int32_t*)(ws + l.wgs);
  a.wg_begin = (const int32_t*)(ws + l.wgb);
  a.seg_w0 = (const int32_t*)(ws + l.sw0);
  a.part_ml = (float*)(ws + l.ml);
  a.part_o = (float*)(ws + l.o);
  pa_status e = launch(prefill_prep_kernel, dim3(1), dim3(1024), 0, st, a, num_seqs, total_q,
                       max_q_len, PF_ROWS / G, W, (int32_t*)(ws + l.hdr), (int32_t*)(ws + l.seq),
                       (int32_t*)(ws + l.seg), (int4*)(ws + l.desc), (int32_t*)(ws + l.wgs),
                       (int32_t*)(ws + l.wgb), (int32_t*)(ws + l.sw0),
                       route ? (int32_t*)(ws + l.drow_ctx) : nullptr,
                       route ? (int32_t*)(ws + l.drow_map) : nullptr);
  if (e == PA_OK) e = launch(prefill_kernel<CDT, HD, G, DIRECT>, dim3(W), dim3(256), 0, st, a);
  if (e == PA_OK)
    e = launch(prefill_merge_kernel<HD, G>, dim3(a.nseg_max * (PF_ROWS / MergeShape<HD>::ROWS)),
               dim3(256), 0, st, a, W);
  return e;
}

// bf16 caches at head_dim 128 with blocks of 16 tokens or more load their
// tiles straight into LDS; the rest stage them through registers (8- and 4-bit
// codes are widened on the way)
template <int CDT, int HD, int G>
static pa_status pf_launch(PrefillArgs a, int num_seqs, int total_q, int max_q_len,
                           const PfLayout& l, char* ws, bool route, hipStream_t st) {
  if constexpr (CDT == PA_BF16 && HD == 128) {
    if (a.block_size >= 16)
      return pf_launch_k<CDT, HD, G, true>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
  }
  return pf_launch_k<CDT, HD, G, false>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
}

template <int CDT, int HD>
static pa_status pf_dispatch_g(int G, const PrefillArgs& a, int num_seqs, int total_q,
                               int max_q_len, const PfLayout& l, char* ws, bool route,
                               hipStream_t st) {
  switch (G) {
    case 1: return pf_launch<CDT, HD, 1>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
    case 2: return pf_launch<CDT, HD, 2>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
    case 4: return pf_launch<CDT, HD, 4>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
    case 8: return pf_launch<CDT, HD, 8>(a, num_seqs, total_q, max_q_len, l, ws, route, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

// Bound on the segments of a batch of num_seqs chunks holding total_q queries,
// none longer than max_q_len: sum_s ceil(L_s / QB) <= (total_q + num_seqs (QB - 1)) / QB
// and <= num_seqs ceil(max_q_len / QB), times the KV heads.
static int64_t pf_nseg_bound(int num_seqs, int total_q, int max_q_len, int n_kv, int G) {
  const int64_t QB = PF_ROWS / G;
  const int64_t by_total = ((int64_t)total_q + (int64_t)num_seqs * (QB - 1)) / QB;
  const int64_t by_max = (int64_t)num_seqs * (((int64_t)max_q_len + QB - 1) / QB);
  return (int64_t)n_kv * (by_total < by_max ? by_total : by_max);
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t max_context_len) {
  (void)max_context_len;
  if (num_seqs <= 0 || total_q <= 0 || max_q_len <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 ||
      n_q_heads % n_kv_heads || head_dim <= 0)
    return 0;
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return 0;
  // the larger of the two plans: matrix-core tiles (bf16 queries) or one
  // decode row per query (fp32 queries and cache)
  const size_t mf = pf_layout(num_seqs, pf_nseg_bound(num_seqs, total_q, max_q_len, n_kv_heads, G),
                              (int64_t)pf_cu_count() * PF_MAX_WGS_PER_CU, head_dim, n_kv_heads,
                              G).total;
  const size_t rows = prefill_f32_workspace_bytes(total_q, n_kv_heads, G, head_dim, max_context_len);
  return mf > rows ? mf : rows;
}

static pa_status prefill_impl(void* out, const void* q, int q_dtype, const int32_t* cu_seqlens_q,
                              int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                              const void* k_cache, const void* v_cache, int cache_dtype,
                              int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                              int32_t head_dim, int32_t group_size, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t max_context_len, int32_t causal, float scale,
                              float k_scale, float v_scale, void* workspace,
                              size_t workspace_bytes, void* stream,
                              const float* k_channel_scales, const float* v_scales) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || n_kv_heads < 1 ||
      max_blocks_per_seq < 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1))) return PA_ERR_UNSUPPORTED;
  if (group_size != 1 && group_size != 2 && group_size != 4 && group_size != 8)
    return PA_ERR_UNSUPPORTED;
  const bool int4 = cache_dtype == PA_INT4;
  const bool f32 = q_dtype == PA_F32 && cache_dtype == PA_F32;
  if (!f32 && (q_dtype != PA_BF16 || (cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3 &&
                                      cache_dtype != PA_INT8 && !int4)))
    return PA_ERR_DTYPE;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !cu_seqlens_q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL;
  if (f32) {
    if (!(scale > 0.0f) || scale > 3.0e38f) return PA_ERR_SHAPE;
    if (!workspace || ((uintptr_t)workspace & 255)) return PA_ERR_WORKSPACE;
    return prefill_f32_rows((float*)out, (const float*)q, cu_seqlens_q, num_seqs, total_q,
                            k_cache, v_cache, num_blocks, block_size, n_kv_heads, head_dim,
                            group_size, block_tables, max_blocks_per_seq, context_lens,
                            max_context_len, causal, scale, workspace, workspace_bytes,
                            (hipStream_t)stream);
  }
  if (int4 && (!k_channel_scales || !v_scales)) return PA_ERR_NULL;
  // 8-bit caches (fp8 or int8) carry per-tensor scales
  const bool fp8 = cache_dtype == PA_FP8_E4M3 || cache_dtype == PA_INT8;
  if (fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f))) return PA_ERR_SHAPE;
  // the kernel takes row maxima of the unscaled scores
  if (!(scale > 0.0f) || scale > 3.0e38f) return PA_ERR_SHAPE;
  const int64_t nseg = pf_nseg_bound(num_seqs, total_q, max_q_len, n_kv_heads, group_size);
  // units (key tiles and start-up units) are counted in 32-bit integers
  // (the merge launches PF_ROWS / 4 workgroups per segment at head_dim 64)
  if (nseg * (PF_ROWS / 4) >= ((int64_t)1 << 31) ||
      nseg * ((int64_t)max_context_len / PF_BN + 1 + PF_OV) >= ((int64_t)1 << 31))
    return PA_ERR_SHAPE;
  const PfLayout l = pf_layout(num_seqs, nseg, (int64_t)pf_cu_count() * PF_MAX_WGS_PER_CU, head_dim,
                               n_kv_heads, group_size);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace & 255)) return PA_ERR_WORKSPACE;
  // a block's rows are addressed with 32-bit offsets
  if ((int64_t)block_size * n_kv_heads * head_dim * 2 >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  PrefillArgs a;
  a.q = (const uint8_t*)q;
  a.out = out;
  a.cu_q = cu_seqlens_q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.tok_stride = (int64_t)n_kv_heads * head_dim * (int4 ? 4 : fp8 ? 8 : 16) / 8;
  a.k_ch_scale = k_channel_scales;
  a.v_tok_scale = v_scales;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  a.bs_log2 = lg;
  a.n_kv = n_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.nseg_max = (int)nseg;
  a.cus = pf_cu_count();
  a.causal = causal != 0;
  a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 ? v_scale : 1.0f;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  pa_status (*dispatch)(int, const PrefillArgs&, int, int, int, const PfLayout&, char*, bool,
                        hipStream_t);
  if (cache_dtype == PA_BF16)
    dispatch = head_dim == 128 ? pf_dispatch_g<PA_BF16, 128> : pf_dispatch_g<PA_BF16, 64>;
  else if (cache_dtype == PA_FP8_E4M3)
    dispatch = head_dim == 128 ? pf_dispatch_g<PA_FP8_E4M3, 128> : pf_dispatch_g<PA_FP8_E4M3, 64>;
  else if (cache_dtype == PA_INT8)
    dispatch = head_dim == 128 ? pf_dispatch_g<PA_INT8, 128> : pf_dispatch_g<PA_INT8, 64>;
  else
    dispatch = head_dim == 128 ? pf_dispatch_g<PA_INT4, 128> : pf_dispatch_g<PA_INT4, 64>;
  // Rows of length 1 (decode rows in the batch) take the decode kernel's path
  // when the blocks allow it (16 tokens or more): whole token rows streamed
  // through the matrix cores, where the tile kernel would give such a row one
  // wave in four and 4 of its 32 query columns.  The planner lists them; the
  // tile kernel skips them.  A batch declared as num_seqs chunks of max_q_len
  // (> 1) queries each has no such row, and then the decode path's launches
  // are not enqueued (about 8 us of empty launches on the mixed step); if its
  // offsets held a row of length 1 after all, the tile kernel computes it.
  const bool route = block_size >= 16 &&
                     !(max_q_len > 1 && (int64_t)total_q == (int64_t)num_seqs * max_q_len);
  // the decode path counts its 16-token units in 32-bit integers; checked here,
  // before anything is enqueued
  if (route && (int64_t)num_seqs * n_kv_heads * (((int64_t)max_context_len + 15) / 16 + DECODE_SEG_OV_MAX) >=
                   ((int64_t)1 << 31))
    return PA_ERR_SHAPE;
  pa_status e = dispatch(group_size, a, num_seqs, total_q, max_q_len, l, ws, route, st);
  if (e != PA_OK || !route) return e;
  return prefill_decode_rows(out, q, k_cache, v_cache, cache_dtype, num_blocks, block_size,
                             n_kv_heads, head_dim, group_size, block_tables, max_blocks_per_seq,
                             (const int32_t*)(ws + l.drow_ctx), (const int32_t*)(ws + l.drow_map),
                             num_seqs, max_context_len, scale, k_scale, v_scale,
                             k_channel_scales, v_scales, ws + l.dws, l.dws_bytes, st);
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
  if (cache_dtype == PA_INT4) return PA_ERR_DTYPE;   // its scales come through pa_prefill_chunk_int4
  return prefill_impl(out, q, q_dtype, cu_seqlens_q, num_seqs, total_q, max_q_len, k_cache,
                      v_cache, cache_dtype, num_blocks, block_size, n_kv_heads, head_dim,
                      group_size, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                      causal, scale, k_scale, v_scale, workspace, workspace_bytes, stream, nullptr,
                      nullptr);
}

extern "C" pa_status pa_prefill_chunk_int4(void* out, const void* q, int q_dtype,
                                           const int32_t* cu_seqlens_q, int32_t num_seqs,
                                           int32_t total_q, int32_t max_q_len,
                                           const void* k_cache, const void* v_cache,
                                           const float* k_channel_scales, const float* v_scales,
                                           int32_t num_blocks, int32_t block_size,
                                           int32_t n_kv_heads, int32_t head_dim,
                                           int32_t group_size, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t max_context_len,
                                           int32_t causal, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return prefill_impl(out, q, q_dtype, cu_seqlens_q, num_seqs, total_q, max_q_len, k_cache,
                      v_cache, PA_INT4, num_blocks, block_size, n_kv_heads, head_dim, group_size,
                      block_tables, max_blocks_per_seq, context_lens, max_context_len, causal,
                      scale, 1.0f, 1.0f, workspace, workspace_bytes, stream, k_channel_scales,
                      v_scales);
}

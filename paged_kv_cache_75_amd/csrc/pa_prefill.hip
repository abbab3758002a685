// Chunked prefill attention for gfx950 (pa_prefill): causal attention of
// each sequence's newest M tokens through its block table, on the matrix
// cores, with K/V rows shared by the waves of a workgroup through LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cfloat>
#include <cstdint>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_launch.h"

namespace pa {

namespace {

// Chunked prefill: causal attention of each sequence's last M tokens (a prompt
// chunk; a decode token is M = 1).  A workgroup of kPrefillWaves waves takes
// one (query block, kv head, sequence); each wave holds kBlocks column blocks,
// each filling the 16 columns of an MFMA operand holding Q^T with 16 / G
// queries times the G heads of the kv head (integer division).  Column c of
// block b of wave w is query r = (w * kBlocks + b) * (16 / G) + c / G of the
// query block (head c % G) at position T - M + r; key rows after that position get weight zero
// (its per-lane `live` bound).
//
// The workgroup walks the keys in 32-key steps up to its last position.  Each
// step's key and value rows are loaded once into LDS, where all the waves'
// column blocks read them: keys as the A operand of S^T = K . Q^T (row-wise
// reads), values through transposed reads for O^T += V^T . P^T (rows padded:
// PrefillLds).  When tiles lie inside blocks the rows go from memory straight
// into LDS (LDS-direct buffer loads: key rows packed, four or eight per
// instruction; value rows one per instruction), and a step's
// P.V products are issued at the start of the next step, ahead of that step's
// softmax reference, so that each wave's matrix and vector work overlap; the
// values are then read a step later, so four LDS stages rotate.  Smaller
// blocks stage the rows through registers, with three stages and P.V in its
// own step.  One barrier per step: a stage is rewritten only after every wave
// has passed the barrier that follows its last reader.
//
// Workgroup order: workgroup i runs on XCD i mod kXcds, and each XCD has its
// own L2.  All query blocks of one (sequence, kv head) pair go to one XCD, a
// pair after another, so the pair's key and value rows, read by every one of
// its query blocks, stay in that XCD's L2.  Pairs are handed out longest
// sequence first (up to kWave sequences; beyond that in index order), and
// within a pair the latest query blocks first: the workgroups with the most
// keys start early instead of forming a tail.  Which workgroup runs a (pair,
// query block) does not change its arithmetic, so the results do not depend
// on it.
// ---------------------------------------------------------------------------
template <int G>
struct PrefillShape {
  static constexpr int kBlockQueries = 16 / G;          // queries per column block
  static constexpr int kBlocks = kPrefillColumnBlocks;  // column blocks per wave
  static constexpr int kQueries = kBlockQueries * kBlocks;
};

// The sequence of rank k when sequences are ordered by clamped length,
// longest first, equal lengths by index (num_seqs <= kWave: lane s holds
// sequence s's length; every workgroup derives the same order).  Binary search
// for the length v of rank k -- the largest v with more than k lengths >= v --
// then the (k - #{lengths > v})-th sequence of length v.
__device__ __forceinline__ int seq_of_rank(const DecodeArgs& a, int k, int& len) {
  const int lane = threadIdx.x % kWave;
  const int key =
      lane < a.num_seqs ? min(max(a.context_lens[lane], 0), a.max_context_len) : -1;
  uint32_t lo = 0, hi = uint32_t(a.max_context_len) + 1;   // count(lo) > k >= count(hi)
  while (hi - lo > 1) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (__popcll(__builtin_amdgcn_ballot_w64(key >= int(mid))) > k) lo = mid;
    else hi = mid;
  }
  const int v = int(lo);
  const int m = k - __popcll(__builtin_amdgcn_ballot_w64(key > v));
  const uint64_t eq = __builtin_amdgcn_ballot_w64(key == v);
  const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(eq >> 32),
                                              __builtin_amdgcn_mbcnt_lo(uint32_t(eq), 0));
  const int s = __ffsll(static_cast<long long>(
                    __builtin_amdgcn_ballot_w64(key == v && below == m))) - 1;
  len = v;
  return s;
}

// Softmax reference of the prefill: a column keeps its reference m until a
// step's maximum exceeds it by more than kRefSlack (log2 units); only then are
// the wave's sums and outputs rescaled (a wave-uniform branch).  The result is
// the same softmax: every weight exp2(s - m) stays at most 2^kRefSlack, well
// inside float32 and bfloat16 range, and the relative precision of the
// weights does not depend on their scale.
constexpr float kRefSlack = 8.0f;

// The maximum over a column's four lanes (gq = 0..3) with gfx950's
// NaN-propagating maximum (scores are finite or -inf here): unlike fmaxf it
// needs no quieting of the values the lane swaps bring in.
__device__ __forceinline__ float column_maximum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Eight element-type ones: the A operand whose product with the weights gives
// every row of the result the column's sum of the weights.
template <int DT> __device__ inline uint4 ones_chunk();
template <> __device__ inline uint4 ones_chunk<PA_BF16>() {
  return make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
}
template <> __device__ inline uint4 ones_chunk<PA_F16>() {
  return make_uint4(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
}

// One 16-column block of a prefill wave: Q^T operand, O^T accumulators, the
// running reference and sum, and the step's weights.  The sum is a product
// on the matrix cores, (all-ones)^T . P^T beside V^T . P^T: every entry of `l`
// holds the column's sum of the same rounded weights that enter P.V, so the
// result is an exact weighted average of the value rows with those weights
// (its rounding error then scales with how far the values lie from the
// result, not with their size), and no vector instruction adds them.
template <int DT, int D>
struct PrefillCols {
  static constexpr int KK = D / 32;            // 32-element chunks of a query row
  static constexpr int NT = D / 16;            // 16-row tiles of O^T
  uint4 qb[KK];
  f32x4 o[NT];
  f32x4 l;
  float m_run;
  float lim;                                   // raw-score bound of the reference test
  float p[8];                                  // keys 4gq + i of each 16-key half
};

// A step is 32 keys: two 16-key tiles (halves).  S^T = K . Q^T per half gives
// lane (gq, c) the scores of keys 4gq .. 4gq+3 of each half for column c;
// those eight weights are, in that order, the lane's B operand of the
// 16x16x32 product O^T += V^T . P^T (the contraction over keys may take them
// in any order, as long as V^T's chunks follow the same order).
template <int DT, int D>
__device__ __forceinline__ void prefill_qk32(const PrefillCols<DT, D>& t,
                                             const KeyRegs<DT, D>& k0, const KeyRegs<DT, D>& k1,
                                             f32x4& s0, f32x4& s1) {
  s0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  s1 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < PrefillCols<DT, D>::KK; ++kk) {
    s0 = mfma_chunk<DT>(k0.k[kk], t.qb[kk], s0);
    s1 = mfma_chunk<DT>(k1.k[kk], t.qb[kk], s1);
  }
}

// A step's softmax for every column block from its raw scores (S^T = K . Q^T
// per half, lane (gq, c) holding keys 4gq .. 4gq+3 of each half; the query
// rows carry the sign of the scale, so `scale` is its magnitude in log2
// units), in two parts.  The reference: each lane's raw maxima (on diagonal
// steps taken again after masking, in place), then one wave-uniform test
// whether any lane's raw maximum exceeds its
// column's bound `lim` (the reference plus kRefSlack, in raw units); only then
// are the column maxima formed and the reference moved, with the rescale.
// The weights: exp2(raw * scale - m) with the scale inside the FMA.  Between
// the two the next step's score products are issued, so that they run on the
// matrix cores while the weights are computed.
template <int DT, int D, int NB, bool kAfterProducts>
__device__ __forceinline__ void prefill_reference(PrefillCols<DT, D> (&cols)[NB], float scale,
                                                  f32x4 (&sc)[NB][2], int gq, bool mask,
                                                  const int (&live)[NB][2]) {
  auto maxima = [&](float (&mx)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float m = sc[b][0][0];
#pragma unroll
      for (int i = 1; i < 4; ++i) m = __builtin_elementwise_maximum(m, sc[b][0][i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) m = __builtin_elementwise_maximum(m, sc[b][1][i]);
      mx[b] = m;
    }
  };
  // The raw maxima come first, ahead of the masking branch, so that they
  // share one scheduling region with the products issued just before (the
  // deferred P.V: kAfterProducts).  There the order is set: eight products
  // back to back (by then the scores of the step before have left the
  // matrix cores), then one product per two vector instructions, then the
  // rest.  Steps on the diagonal mask and take the maxima again.
  float mx[NB];
  maxima(mx);
  if constexpr (kAfterProducts) {
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // matrix products
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0); // vector instructions
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  }
  if (mask) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * gq + i >= live[b][0]) sc[b][0][i] = -INFINITY;
        if (4 * gq + i >= live[b][1]) sc[b][1][i] = -INFINITY;
      }
    maxima(mx);
  }
  bool move = false;
#pragma unroll
  for (int b = 0; b < NB; ++b) move |= mx[b] > cols[b].lim;
  if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      PrefillCols<DT, D>& t = cols[b];
      // scaling is monotonic (scale > 0): the column's maximum of the scaled
      // scores; -inf when nothing is live yet
      const float cm = column_maximum(mx[b]) * scale;
      const float m_new = fmaxf(t.m_run, cm);
      // a column with nothing so far (m_new = -inf) has nothing to rescale
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(t.m_run - m_new);
#pragma unroll
      for (int n = 0; n < PrefillCols<DT, D>::NT; ++n) t.o[n] *= alpha;
      t.l *= alpha;
      t.m_run = m_new;
      // raw scores above this take a weight above 2^kRefSlack
      t.lim = m_new == -INFINITY ? -INFINITY : (m_new + kRefSlack) / scale;
    }
  }
}

// A masked key's raw score is -inf, so its exponent is -inf and its weight 0
// (the scale is at least FLT_MIN, never 0).
template <int DT, int D, int NB>
__device__ __forceinline__ void prefill_weights(PrefillCols<DT, D> (&cols)[NB], float scale,
                                                const f32x4 (&sc)[NB][2]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    PrefillCols<DT, D>& t = cols[b];
    const float m_use = t.m_run == -INFINITY ? 0.0f : t.m_run;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t.p[i] = __builtin_amdgcn_exp2f(fmaf(sc[b][0][i], scale, -m_use));
      t.p[4 + i] = __builtin_amdgcn_exp2f(fmaf(sc[b][1][i], scale, -m_use));
    }
  }
}

// LDS rows of a prefill step, key and value rows both padded by 32 bytes.
// The LDS serves 32 lanes per pass from 128 four-byte banks; with a row
// stride of 72 (or 40) words, 16 consecutive rows start on 16 distinct
// multiples of 8 banks, so a key read (16 bytes of 16 rows for 32 lanes) and
// a transposed value read (32 bytes of 8 rows for 32 lanes) find no conflict,
// and every read address is a per-lane base plus a constant.  The staging
// writes take rows r, r + 8 (r, r + 4, r + 8, r + 12 for 128-byte rows) in
// one pass, whose 256-byte spans are disjoint modulo 512 bytes.
//
// Packed keys (rows straight from memory): key rows unpadded, the 16-byte
// chunks of row r rotated, chunk ch stored at (ch + 2r) mod kChunks: the same
// 32-byte shift per row that the padding gives, inside the row.  The bank
// counter reads no conflict for it (XOR permutations of the chunks left
// conflicts).  A 16-byte LDS-direct load fills four (eight) whole rows: each
// lane fetches the memory chunk its LDS place holds.
template <int DT, int D, bool kPackedKeys = false>
struct PrefillLds {
  static constexpr int kRowBytes = Geo<DT, D, 16>::kRowBytes;
  static constexpr int kKeyStride = kPackedKeys ? kRowBytes : kRowBytes + 32;
  static constexpr int kValStride = kRowBytes + 32;
  static constexpr int kStepRows = 2 * kTileTokens;
  static constexpr int kValOffset = kStepRows * kKeyStride;
  static constexpr int kStageBytes = kValOffset + kStepRows * kValStride;
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks of a row
};
// A 16-byte-per-lane LDS-direct load (gfx950): lane l's 16 bytes at dst + 16 l.
// (A device function of its own: the host compilation pass, which checks the
// builtin's size against no gfx950 target, never sees the call.)
__device__ __forceinline__ void lds_direct_load16(__amdgpu_buffer_rsrc_t r, lds_char* dst,
                                                  int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voffset, 0, 0, 0);
}
// The packed-key place of memory chunk ch of step row r, and the memory
// chunk at place p.
template <int DT, int D>
__device__ __forceinline__ int key_place(int r, int ch) {
  return (ch + 2 * r) & (PrefillLds<DT, D, true>::kChunks - 1);
}
template <int DT, int D>
__device__ __forceinline__ int key_chunk_at(int r, int p) {
  return (p - 2 * r) & (PrefillLds<DT, D, true>::kChunks - 1);
}

// O^T += V^T . P^T over a 32-key step for every column block, in two parts:
// read_v32 reads the A operand chunks, accumulate32 does the products.  The
// step's 32 value rows sit in LDS at the padded stride; `rbase` points at
// lane (gq, c)'s first read: row 4gq + c/4 of the first half, dimensions
// 4(c%4) .. +3.  A transposed read gives the lane four keys of one
// dimension, 4gq .. 4gq+3 of a half, and the read 16 rows further on the
// same four keys of the second half: together the A operand chunk matching
// the weights' order.
template <int DT, int D, int NT>
__device__ __forceinline__ void read_v32(uint4 (&av)[NT], lds_char* rbase) {
  constexpr int kValStride = PrefillLds<DT, D>::kValStride;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    lds_char* at = rbase + 32 * n;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)at);
    const v4i16 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(at + kTileTokens * kValStride));
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    av[n] = make_uint4(l.x, l.y, h.x, h.y);
  }
}
// The step's weights of every column block as B operand chunks (rounded to
// the element type), and the products with the value chunks `avs` (and with
// all-ones for the sums).
template <int DT, int D, int NB>
__device__ __forceinline__ void pack_weights(const PrefillCols<DT, D> (&cols)[NB], uint4 (&pb)[NB]) {
  // two four-element halves as one eight-element operand chunk
  auto join = [](v4i16 lo, v4i16 hi) {
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    return make_uint4(l.x, l.y, h.x, h.y);
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) pb[b] = join(pack4<DT>(cols[b].p), pack4<DT>(cols[b].p + 4));
}
template <int DT, int D, int NB, int NT>
__device__ __forceinline__ void accumulate_packed(PrefillCols<DT, D> (&cols)[NB], const uint4 (&avs)[NT],
                                                  const uint4 (&pb)[NB]) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint4 av = avs[n];
#pragma unroll
    for (int b = 0; b < NB; ++b) cols[b].o[n] = mfma_chunk<DT>(av, pb[b], cols[b].o[n]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) cols[b].l = mfma_chunk<DT>(ones_chunk<DT>(), pb[b], cols[b].l);
}
template <int DT, int D, int NB, int NT>
__device__ __forceinline__ void accumulate32(PrefillCols<DT, D> (&cols)[NB], const uint4 (&avs)[NT]) {
  uint4 pb[NB];
  pack_weights<DT, D, NB>(cols, pb);
  accumulate_packed<DT, D, NB, NT>(cols, avs, pb);
}

template <int DT, int D, int G, bool kTileInBlock>
__global__ __launch_bounds__(kWave * kPrefillWaves, 2) void prefill_kernel(DecodeArgs a) {
  using GE = Geo<DT, D, 16>;
  constexpr int KK = GE::KK, CPR = GE::CPR;
  constexpr int kRowBytes = GE::kRowBytes;
  constexpr int BQ = PrefillShape<G>::kBlockQueries;
  constexpr int NB = PrefillShape<G>::kBlocks;
  constexpr int QW = PrefillShape<G>::kQueries;          // queries per wave
  constexpr int QG = QW * kPrefillWaves;                  // queries per workgroup
  constexpr int kThreads = kWave * kPrefillWaves;
  constexpr int kStepRows = 2 * kTileTokens;              // keys per step
  constexpr int kLoadRows = kThreads / CPR;               // rows per load instruction
  constexpr int kLoads = kStepRows / kLoadRows;           // per matrix and step
  using LS = PrefillLds<DT, D, kTileInBlock>;
  constexpr int kStageBytes = LS::kStageBytes;            // keys, then values
  // Tiles inside blocks: a step's P.V waits for the next step (deferred), so
  // a stage is read until the step after its own and four stages rotate.
  constexpr bool kDeferPV = kTileInBlock;
  constexpr int kStages = kDeferPV ? 4 : 3;
  static_assert(kThreads % CPR == 0 && kStepRows % kLoadRows == 0 &&
                    (kLoadRows % kTileTokens == 0 || kTileTokens % kLoadRows == 0),
                "load shape");
  using PC = PrefillCols<DT, D>;
  __shared__ __align__(16) char lds[kStages * kStageBytes];

  const int nqb = (a.max_query_len - 1) / QG + 1;          // query blocks per pair (>= 1)
  const int xcd = blockIdx.x % kXcds;
  const int j = blockIdx.x / kXcds;                         // this XCD's j-th workgroup
  const int pair = xcd + kXcds * (j / nqb);                 // pair rank
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int rank = pair / a.num_kv_heads;
  const int g = pair - rank * a.num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  int T, seq;
  if (a.num_seqs <= kWave) {
    seq = seq_of_rank(a, rank, T);
  } else {
    seq = rank;
    T = min(max(a.context_lens[seq], 0), a.max_context_len);
  }
  const int row_begin = a.query_start[seq];
  const int M = min(max(a.query_start[seq + 1] - row_begin, 0), T);
  const int r0 = (nqb - 1 - j % nqb) * QG;                 // latest query blocks first
  if (r0 >= M) return;                                      // the whole workgroup
  const int nq_wg = min(QG, M - r0);
  const int rw = r0 + wave * QW;                            // this wave's first query
  const int nq = max(0, min(QW, M - rw));

  PC cols[NB];
  const int gq = lane >> 4, c = lane & 15;
  const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  // a zero scale is taken as FLT_MIN: every finite score times it rounds
  // away against the reference, so the weights are the same (all 1 before
  // normalisation), and a masked key's -inf stays -inf instead of NaN
  const float scale = fmaxf(fabsf(a.scale_log2), FLT_MIN);
  bool col_ok[NB];
  int pos[NB];
  int64_t out_row[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    col_ok[b] = b * BQ + c / G < nq && c < BQ * G;
    const int qr = rw + (col_ok[b] ? b * BQ + c / G : 0);   // query row of this column
    const int head = g * G + (col_ok[b] ? c % G : 0);
    pos[b] = T - M + qr;                                      // its position
    out_row[b] = int64_t(row_begin + min(qr, M - 1)) * a.num_q_heads + head;
    const uint4* qrow = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                       out_row[b] * kRowBytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 v = col_ok[b] ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
      // the scale's sign moves into the query (exact: a sign flip)
      cols[b].qb[kk] = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
    }
#pragma unroll
    for (int n = 0; n < PC::NT; ++n) cols[b].o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    cols[b].l = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    cols[b].m_run = -INFINITY;
    cols[b].lim = -INFINITY;
  }

  // the wave's first position; a wave with no queries computes columns it
  // never stores, so any bound serves it
  const int first_pos = T - M + rw;
  // steps this wave computes: up to its last query's position (none when it
  // holds no query rows, e.g. the decode tokens of a mixed batch).  Later
  // steps are wholly masked for it and would leave its sums unchanged; the
  // wave still stages rows and meets every barrier.
  const int wave_steps = nq > 0 ? ((T - M + rw + nq - 1) / kTileTokens + 2) / 2 : 0;
  const int ntiles = (T - M + r0 + nq_wg - 1) / kTileTokens + 1;   // up to the last position
  const int nsteps = (ntiles + 1) / 2;                             // 32-key steps
  const int lb = a.log2_block;
  const int bmask = (1 << lb) - 1;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq;
  const int64_t head_rows = int64_t(g) << lb;
  const int64_t blk_rows = int64_t(a.num_kv_heads) << lb;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int nblk = a.num_blocks;
  // this thread's share of a step: chunk lchunk of step rows lrow + i * kLoadRows,
  // the rows of one 32-lane pass spread as the LDS layout wants
  constexpr int kPassRows = 32 / CPR;
  const int q = threadIdx.x / CPR, lchunk = threadIdx.x % CPR;
  const int lrow = (q & ~15) + (q & 15) / kPassRows + (16 / kPassRows) * (q % kPassRows);
  // the tile a load instruction of this wave covers, relative to the step's
  // first tile (the same for all of the wave's lanes)
  auto load_half = [&](int i) {
    return (i * kLoadRows + wave * (kWave / CPR)) / kTileTokens;
  };

  // tile k's block (one per lane, 64 tiles per load) when tiles lie in blocks
  int tbl = 0;
  auto load_tbl = [&](int batch) {
    const int k = min(64 * batch + lane, ntiles - 1);
    tbl = min(max(table[(k * kTileTokens) >> lb], 0), nblk - 1);
  };
  // the buffer spans the tile's rows below T only; a tile past the last
  // position (the second half of the last step) spans none: its table lane
  // holds another tile's block, and it must read as zeros
  auto rsrc = [&](const char* base, int k) {
    const int64_t blk = __builtin_amdgcn_readlane(tbl, k & 63);
    const int64_t byte = (blk * blk_rows + head_rows + ((k * kTileTokens) & bmask)) * kRowBytes;
    const int rows = k < ntiles ? min(kTileTokens, T - k * kTileTokens) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + byte), 0,
                                             rows * kRowBytes, kBufferDword3);
  };
  // blocks smaller than a tile: each row finds its block; rows past T - 1
  // read row T - 1 (weight zero)
  auto row_of = [&](int t) -> int64_t {
    t = min(t, T - 1);
    const int64_t blk = min(max(table[t >> lb], 0), nblk - 1);
    return blk * blk_rows + head_rows + (t & bmask);
  };
  // tiles inside blocks: the rows of step st go from memory straight into
  // LDS stage st % kStages (rows past T, and a tile past the last position,
  // read as zeros).  Wave w moves step rows 8w .. 8w + 7 of the keys and of
  // the values, which lie in one tile: the keys 16 bytes a lane, whole rows
  // per load in their packed, rotated place; the values 4 bytes a lane, one
  // row per load at its padded place.
  constexpr int kRowsPerWave = kStepRows / kPrefillWaves;
  constexpr int kRowLanes = kRowBytes / 4;
  constexpr int kKeyRowsPerLoad = kWave / LS::kChunks;
  constexpr int kKeyLoads = kRowsPerWave / kKeyRowsPerLoad;
  static_assert(kRowsPerWave * kPrefillWaves == kStepRows && kTileTokens % kRowsPerWave == 0 &&
                    kRowLanes <= kWave && kRowsPerWave % kKeyRowsPerLoad == 0,
                "direct row loads");
  // this lane's memory offset, within its tile, for each packed key load:
  // row r0 + i * kKeyRowsPerLoad + lane / kChunks, the chunk whose place is
  // chunk lane % kChunks of that row
  int key_off[kKeyLoads];
#pragma unroll
  for (int i = 0; i < kKeyLoads; ++i) {
    const int sr = wave * kRowsPerWave + i * kKeyRowsPerLoad + lane / LS::kChunks;
    const int ch = key_chunk_at<DT, D>(sr, lane % LS::kChunks);
    key_off[i] = (sr % kTileTokens) * kRowBytes + 16 * ch;
  }
  // byte offset of step st's LDS stage, unsigned so that the compiler can
  // fold each read's constant part into the instruction's offset field
  auto stage_of = [](int st) -> uint32_t { return uint32_t(st) % kStages * kStageBytes; };
  auto load_rows = [&](int st) {
    const int r0 = wave * kRowsPerWave;
    const int k = 2 * st + r0 / kTileTokens;
    const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, k), rv = rsrc(vbase, k);
    lds_char* const sb = (lds_char*)lds + stage_of(st);
#pragma unroll
    for (int i = 0; i < kKeyLoads; ++i)
      lds_direct_load16(rk, sb + (r0 + i * kKeyRowsPerLoad) * LS::kKeyStride, key_off[i]);
    if (lane < kRowLanes) {
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        const int sr = r0 + i;
        const int off = (sr % kTileTokens) * kRowBytes + 4 * lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, sb + LS::kValOffset + sr * LS::kValStride, 4,
                                                 off, 0, 0, 0);
      }
    }
  };
  // every wave's rows in LDS before the barrier that lets the others read them
  auto rows_landed = [] { __builtin_amdgcn_s_waitcnt(0x0f70); };   // vmcnt(0)
  // blocks smaller than a tile: staged through registers
  struct Stage {
    uint4 k[kLoads], v[kLoads];
  };
  auto load_step = [&](int st, Stage& r) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int sr = i * kLoadRows + lrow;                 // row of the step
      const int64_t row = row_of(st * kStepRows + sr);
      r.k[i] = reinterpret_cast<const uint4*>(kbase + row * kRowBytes)[lchunk];
      r.v[i] = reinterpret_cast<const uint4*>(vbase + row * kRowBytes)[lchunk];
    }
  };
  auto store_step = [&](const Stage& r, char* st) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int sr = i * kLoadRows + lrow;
      *reinterpret_cast<uint4*>(st + sr * LS::kKeyStride + lchunk * 16) = r.k[i];
      *reinterpret_cast<uint4*>(st + LS::kValOffset + sr * LS::kValStride + lchunk * 16) =
          r.v[i];
    }
  };

  Stage R;
  // lane (gq, c) reads value row 4gq + c/4, dimensions 16n + 4(c%4) .. +3 of
  // each step (a local-memory pointer: stage and constants fold into the
  // read instructions' offsets)
  lds_char* const lds_v = (lds_char*)lds + LS::kValOffset +
                          (4 * gq + (c >> 2)) * LS::kValStride + ((c & 1) << 3) +
                          (((c & 3) >> 1) << 4);
  // S^T of a step for every column block: the key fragments from the step's
  // LDS stage (lane (gq, c): key row c of each half, chunks 4kk + gq), then
  // the products
  using Scores = f32x4[NB][2];
  using Keys = KeyRegs<DT, D>[2];
  // lane (gq, c) reads key row c of each half, chunks 4kk + gq (packed keys:
  // at their rotated places, the same in both halves: 2 (c + 16) = 2c modulo
  // the chunks of a row)
  int key_rd[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    key_rd[kk] = c * LS::kKeyStride +
                 16 * (kTileInBlock ? key_place<DT, D>(c, 4 * kk + gq) : 4 * kk + gq);
  auto read_k = [&](int st, Keys& kr) {
    const char* kb = lds + __builtin_amdgcn_readfirstlane(stage_of(st));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kr[h].k[kk] =
            *reinterpret_cast<const uint4*>(kb + key_rd[kk] + h * kTileTokens * LS::kKeyStride);
  };
  auto qk = [&](const Keys& kr, Scores& sc) {
#pragma unroll
    for (int b = 0; b < NB; ++b) prefill_qk32<DT, D>(cols[b], kr[0], kr[1], sc[b][0], sc[b][1]);
  };
  // Step st.  After the barrier every stage up to st + 1 is complete: the
  // wave reads this step's value fragments and the next step's key
  // fragments, only then requests the rows of step st + 2 (into the stage
  // step st - 1 used, which every wave has left), and computes: step st's
  // softmax reference, step st + 1's score products, the weights and P.V
  // (`cur` holds step st's scores, `next` receives step st + 1's).  With
  // blocks smaller than a tile the rows of step st + 1 are staged from
  // registers before the barrier instead.
  //
  // Deferred P.V (tiles inside blocks): step st issues the products of step
  // st - 1's weights (held packed in pb) with that step's values first, then
  // its own softmax reference on the vector units while the matrix cores
  // work, so one wave overlaps the two.  The sums are the same and in the
  // same order: step st - 1's products are added before step st may rescale.
  // A wave computes one step past its last (wholly masked: its weights are
  // zero) to add its last products, or adds them after the loop when that
  // step is the workgroup's last; at step 0 the held weights are zero and
  // the values read are step 0's.
  uint4 pb[NB] = {};
  const int compute_steps =
      kDeferPV ? (wave_steps > 0 ? min(wave_steps + 1, nsteps) : 0) : wave_steps;
  auto step = [&](int st, Scores& cur, Scores& next) {
    if constexpr (kTileInBlock) {
      rows_landed();
    } else if (st + 1 < nsteps) {
      store_step(R, lds + stage_of(st + 1));
      if (st + 2 < nsteps) load_step(st + 2, R);
    }
    __syncthreads();
    const bool computes = st < compute_steps;
    Keys kr;
    uint4 avs[PC::NT];
    if (computes) {
      // the values of this step (of the step before, deferred: read first,
      // as the first products use them), the next step's keys (past the last
      // step: whatever the stage holds, unused)
      const int vs = kDeferPV ? (st > 0 ? st - 1 : 0) : st;
      read_v32<DT, D, PC::NT>(avs, lds_v + __builtin_amdgcn_readfirstlane(stage_of(vs)));
      read_k(st + 1, kr);
    }
    if constexpr (kTileInBlock) {
      if (st + 2 < nsteps) {
        if (((2 * st + 4) & 63) == 0) load_tbl((2 * st + 4) >> 6);
        load_rows(st + 2);
      }
    }
    if (!computes) return;
    // masking is needed unless every key of the step precedes every
    // column's position
    const bool mask = (st + 1) * kStepRows - 1 > first_pos;
    int live[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // keys at positions 32 st .. pos of this column take part
      const int before = col_ok[b] ? pos[b] - st * kStepRows + 1 : 0;
      live[b][0] = min(kTileTokens, max(0, before));
      live[b][1] = min(kTileTokens, max(0, before - kTileTokens));
    }
    if constexpr (kDeferPV) {
      accumulate_packed<DT, D, NB, PC::NT>(cols, avs, pb);
      prefill_reference<DT, D, NB, true>(cols, scale, cur, gq, mask, live);
      qk(kr, next);
      prefill_weights<DT, D, NB>(cols, scale, cur);
      pack_weights<DT, D, NB>(cols, pb);
      // the next step's score products spread evenly through the weights:
      // one product per two vector instructions (the compiler's own order
      // left most products at the end, after the exponentials)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // vector instructions
      }
    } else {
      prefill_reference<DT, D, NB, false>(cols, scale, cur, gq, mask, live);
      qk(kr, next);
      prefill_weights<DT, D, NB>(cols, scale, cur);
      accumulate32<DT, D, NB, PC::NT>(cols, avs);
    }
  };

  if constexpr (kTileInBlock) {
    load_tbl(0);
    load_rows(0);
    if (nsteps > 1) load_rows(1);
    rows_landed();
  } else {
    load_step(0, R);
    store_step(R, lds);
    if (nsteps > 1) load_step(1, R);
  }
  __syncthreads();
  Scores SA, SB;
  if (wave_steps > 0) {
    Keys k0;
    read_k(0, k0);
    qk(k0, SA);
  }
  for (int st = 0; st < nsteps; st += 2) {
    step(st, SA, SB);
    if (st + 1 >= nsteps) break;
    step(st + 1, SB, SA);
  }
  if constexpr (kDeferPV) {
    // the last step's products, when that step is the workgroup's last
    if (wave_steps > 0 && wave_steps == nsteps) {
      uint4 avs[PC::NT];
      read_v32<DT, D, PC::NT>(avs, lds_v + __builtin_amdgcn_readfirstlane(stage_of(nsteps - 1)));
      accumulate_packed<DT, D, NB, PC::NT>(cols, avs, pb);
    }
  }

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float l = cols[b].l[0];
    if (col_ok[b]) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int n = 0; n < PC::NT; ++n)
        store4<DT>(a.out, out_row[b] * D + 16 * n + 4 * gq, cols[b].o[n] * inv);
    }
  }
}

}  // namespace

namespace {

template <int DT, int D, int G>
hipError_t launch_prefill_g(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (DT == PA_F32) {
    return hipErrorInvalidValue;
  } else {
    const dim3 grid(static_cast<uint32_t>(
        prefill_workgroups(a.num_seqs, a.num_kv_heads, G, a.max_query_len)));
    if (a.log2_block >= 4)
      launch_timed(prefill_kernel<DT, D, G, true>, grid, dim3(kWave * kPrefillWaves), stream, a);
    else
      launch_timed(prefill_kernel<DT, D, G, false>, grid, dim3(kWave * kPrefillWaves), stream, a);
    return hipGetLastError();
  }
}

template <int DT, int D>
hipError_t launch_prefill_d(const DecodeArgs& a, int32_t group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_g<DT, D, 1>(a, stream);
    case 2: return launch_prefill_g<DT, D, 2>(a, stream);
    case 3: return launch_prefill_g<DT, D, 3>(a, stream);
    case 4: return launch_prefill_g<DT, D, 4>(a, stream);
    case 5: return launch_prefill_g<DT, D, 5>(a, stream);
    case 6: return launch_prefill_g<DT, D, 6>(a, stream);
    case 7: return launch_prefill_g<DT, D, 7>(a, stream);
    case 8: return launch_prefill_g<DT, D, 8>(a, stream);
    case 16: return launch_prefill_g<DT, D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_prefill_dt(const DecodeArgs& a, int32_t head_dim, int32_t group,
                             hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_prefill_d<DT, 64>(a, group, stream);
    case 128: return launch_prefill_d<DT, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const DecodeArgs& a, int32_t dtype, int32_t head_dim, int32_t group,
                          hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  switch (dtype) {
    case PA_F16: return launch_prefill_dt<PA_F16>(a, head_dim, group, stream);
    case PA_BF16: return launch_prefill_dt<PA_BF16>(a, head_dim, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa

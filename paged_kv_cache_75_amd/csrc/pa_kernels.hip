// HIP kernels for gfx950 (CDNA4): the paged KV slot write and paged decode
// attention with a log-sum-exp merge of context partitions.
//
// Address rule ("vLLM Framework and Inference Engine Design", section "What is
// the essence of vLLM's PagedAttention?"): token t of a sequence is in physical
// block table[t >> log2B] at offset t & (B-1).  Pools are
// [num_blocks][num_kv_heads][B][D]: one (block, kv head) pair is B*D
// contiguous elements, so every row of D elements is read with 16-byte loads.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_launch.h"

namespace pa {

namespace {

// fixed partitions: four waves share one partition (the balanced split runs
// one wave per workgroup: each wave is its own share of the work)
constexpr int kPartitionWaves = 4;
constexpr int kMergeThreads = 256;

// ---------------------------------------------------------------------------
// slot write
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void write_kv_kernel(WriteArgs a) {
  const int n = blockIdx.x;
  const int32_t slot = a.slot_mapping[n];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.log2_block;
  const int64_t off = slot & ((1 << a.log2_block) - 1);
  const int chunks_per_row = a.row_bytes / 16;
  const int per_pool = a.num_kv_heads * chunks_per_row;
  for (int c = threadIdx.x; c < 2 * per_pool; c += blockDim.x) {
    const bool is_v = c >= per_pool;
    const int cc = is_v ? c - per_pool : c;
    const int h = cc / chunks_per_row;
    const int ch = cc - h * chunks_per_row;
    const char* src = static_cast<const char*>(is_v ? a.v : a.k) +
                      (int64_t(n) * a.num_kv_heads + h) * a.row_bytes;
    char* dst = static_cast<char*>(is_v ? a.v_pool : a.k_pool) +
                ((blk * a.num_kv_heads + h) << a.log2_block | off) * a.row_bytes;
    reinterpret_cast<uint4*>(dst)[ch] = reinterpret_cast<const uint4*>(src)[ch];
  }
}

// FP8 pools: E4M3 code of a float32 value y = x / scale, rounded to nearest
// with ties to an even mantissa; 448 and above (infinities too) saturate to
// 448, NaN stays NaN.  Written from the OCP 8-bit floating point definition:
// 4 exponent bits with bias 7, 3 mantissa bits, S.1111.111 reserved for NaN.
// a 16-bit element's bits as float (exact)
template <int DT> __device__ inline float half_bits_to_float(uint32_t h);
template <> __device__ inline float half_bits_to_float<PA_F16>(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
template <> __device__ inline float half_bits_to_float<PA_BF16>(uint32_t h) {
  return __uint_as_float(h << 16);
}

// E4M3 (OCP) codes of four floats, packed in a word, the first in the low
// byte: round to nearest even, magnitudes above 448 (infinity included)
// saturate to 448, NaN gives code 0x7f with its sign.  The conversion
// instruction rounds every finite value below 448 exactly so, but does not
// saturate and sets a NaN's sign differently: magnitudes above 448 are
// clamped before it and NaN codes are set after it.  (Compared with the
// definition written out bit by bit over every float bit pattern: no
// difference.)
__device__ inline float e4m3_clamp(float y) {
  const uint32_t u = __float_as_uint(y), mag = u & 0x7fffffffu;
  return (mag > 0x43e00000u && mag <= 0x7f800000u)
             ? __uint_as_float((u & 0x80000000u) | 0x43e00000u)
             : y;
}
__device__ inline uint32_t e4m3_codes4(float y0, float y1, float y2, float y3) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s zero = {0, 0};
  const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, e4m3_clamp(y0), e4m3_clamp(y1),
                                                          1.0f, false);
  const v2s all = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, e4m3_clamp(y2), e4m3_clamp(y3),
                                                           1.0f, true);
  uint32_t w = __builtin_bit_cast(uint32_t, all);
  const float y[4] = {y0, y1, y2, y3};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = __float_as_uint(y[e]);
    if ((u & 0x7fffffffu) > 0x7f800000u)
      w = (w & ~(0xffu << (8 * e))) | ((((u >> 24) & 0x80u) | 0x7fu) << (8 * e));
  }
  return w;
}

// Slot write into FP8 pools: one workgroup per new token, four elements per
// thread (one 32-bit store of codes).
template <int DT>
__global__ __launch_bounds__(256) void write_kv_fp8_kernel(WriteArgs a, float k_scale,
                                                          float v_scale) {
  const int n = blockIdx.x;
  const int32_t slot = a.slot_mapping[n];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.log2_block;
  const int64_t off = slot & ((1 << a.log2_block) - 1);
  const int D = a.row_bytes;                     // FP8 pools: row bytes = head_dim
  const int quads = a.num_kv_heads * D / 4;
  for (int c = threadIdx.x; c < 2 * quads; c += blockDim.x) {
    const bool is_v = c >= quads;
    const int cc = is_v ? c - quads : c;
    const int h = cc / (D / 4);
    const int e0 = (cc - h * (D / 4)) * 4;
    const int64_t src = (int64_t(n) * a.num_kv_heads + h) * D + e0;
    const void* x = is_v ? a.v : a.k;
    const float scale = is_v ? v_scale : k_scale;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float f;
      if constexpr (DT == PA_F32) {
        f = static_cast<const float*>(x)[src + e];
      } else if constexpr (DT == PA_F16) {
        f = static_cast<float>(static_cast<const _Float16*>(x)[src + e]);
      } else {
        f = __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[src + e]) << 16);
      }
      y[e] = f / scale;
    }
    const uint32_t word = e4m3_codes4(y[0], y[1], y[2], y[3]);
    char* dst = static_cast<char*>(is_v ? a.v_pool : a.k_pool) +
                ((blk * a.num_kv_heads + h) << a.log2_block | off) * D + e0;
    *reinterpret_cast<uint32_t*>(dst) = word;
  }
}

// Appending decode: copy row (i, h) of new_k / new_v to token T_i - 1 of
// sequence i, through its block table (lengths clamped as in the decode).
// Sequences with no tokens and table entries outside the pool are skipped.
// Work item j (from `first`, step `stride`) moves one 16-byte chunk.
__device__ void append_rows(const DecodeArgs& a, int row_bytes, int64_t first, int64_t stride) {
  const int cpr = row_bytes / 16;
  const int Hkv = a.num_kv_heads;
  const int64_t per_pool = int64_t(a.num_seqs) * Hkv * cpr;
  for (int64_t j = first; j < 2 * per_pool; j += stride) {
    const bool is_v = j >= per_pool;
    const int64_t jj = is_v ? j - per_pool : j;
    const int64_t row = jj / cpr;                 // i * Hkv + h
    const int ch = int(jj - row * cpr);
    const int i = int(row / Hkv);
    const int h = int(row - int64_t(i) * Hkv);
    const int T = min(a.context_lens[i], a.max_context_len);
    if (T <= 0) continue;
    const int t = T - 1;
    const int32_t blk = a.block_tables[int64_t(i) * a.max_blocks_per_seq + (t >> a.log2_block)];
    if (blk < 0 || blk >= a.num_blocks) continue;
    const int64_t dst_row =
        ((int64_t(blk) * Hkv + h) << a.log2_block) | (t & ((1 << a.log2_block) - 1));
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const char*>(is_v ? a.new_v : a.new_k) + row * row_bytes);
    uint4* dst = reinterpret_cast<uint4*>(
        static_cast<char*>(const_cast<void*>(is_v ? a.v_pool : a.k_pool)) + dst_row * row_bytes);
    dst[ch] = src[ch];
  }
}

__global__ __launch_bounds__(256) void append_kv_kernel(DecodeArgs a, int row_bytes) {
  append_rows(a, row_bytes, int64_t(blockIdx.x) * blockDim.x + threadIdx.x,
              int64_t(gridDim.x) * blockDim.x);
}

// ---------------------------------------------------------------------------
// decode
//
// The work of one (sequence, kv head) pair is cut into 16-token tiles.  A
// workgroup of 4 waves attends over a contiguous run of tiles of one pair (a
// segment); wave w takes tiles w, w+4, w+8, ...
//   K side: lane (gq = lane/16, c = lane%16) loads 16-byte chunks gq, gq+4, ...
//     of token c's key row: the B operand of 16x16 MFMAs whose A operand holds
//     the pair's G query heads repeated down the 16 rows, so lane (gq, c) ends
//     up with token c's scores for four heads.
//   V side: lane (rho = lane/CPR, chi = lane%CPR) loads chunk chi of value rows
//     rho, rho+RPI, ...; it accumulates G x (elements per chunk) float sums.
//   Probabilities pass from the K layout to the V layout through a small LDS
//   tile per wave.
// Online softmax runs in the exp2 domain (scores pre-multiplied by log2 e):
// m = running max, l = running sum of 2^(s - m).  The loads of a wave's next
// tile are in flight while it computes the current one.
// ---------------------------------------------------------------------------
// Sliding window ("vLLM Framework and Inference Engine Design", section on
// sliding windows): a decoded token attends to the last `window` tokens, the
// newest included; window 0 attends to every token.  First position, and the
// 16-token tiles from the one holding it to the end of the sequence.
__device__ inline int window_first(int T, int window) {
  return window > 0 ? max(0, T - window) : 0;
}
__device__ inline int attended_tiles(int T, int window) {
  return T > 0 ? (T + kTileTokens - 1) / kTileTokens - window_first(T, window) / kTileTokens : 0;
}

// Value rows before the window's first position (in the tile holding it) are
// zeroed: their weight is zero, and zero times a non-finite stale value would
// not be.  Lane (rho, chi) holds rows rho, rho + RPI, ...
template <int DT, int D>
__device__ inline void clear_rows_below(ValRegs<DT, D>& v, int first, int rho) {
  constexpr int RPI = Geo<DT, D, 1>::RPI, VS = Geo<DT, D, 1>::VS;
#pragma unroll
  for (int s = 0; s < VS; ++s)
    if (rho + s * RPI < first) v.v[s] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Tile math for 16-bit elements: both products on the matrix cores.
//   Scores transposed, S^T = K . Q^T: A = the key tile (row = token c, as
//   loaded), B = Q^T (column = query head c; columns >= G are zero).  Lane
//   (gq, c) gets tokens 4gq..4gq+3 of head c, so the softmax of a head lives
//   in the four lanes c, c+16, c+32, c+48.
//   Output transposed, O^T += V^T . P^T: B = P^T is exactly the lane's four
//   probabilities (rounded to the element type); A = V^T comes from the
//   wave's V tile in LDS through the gfx950 transpose read, which hands lane
//   (gq, r) the values V[4gq..4gq+3][16n + r].  V rows are stored with their
//   16-byte chunks XOR-swizzled per row so that neither the row writes nor the
//   transposed reads hit the same LDS bank twice.
// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) codes to the compute type, exactly: the gfx950 conversion
// instruction turns the two codes in the low 16 bits of a word into two
// bf16 / fp16 values (checked against the E4M3 definition for all 256 codes).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int DT> __device__ inline uint32_t fp8x2_to(uint32_t w);
template <> __device__ inline uint32_t fp8x2_to<PA_BF16>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <> __device__ inline uint32_t fp8x2_to<PA_F16>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
// codes 8h .. 8h+7 of a 16-code chunk as eight 16-bit values (one MFMA chunk)
template <int DT> __device__ inline uint4 fp8x8_to(const uint4& c, int h) {
  const uint32_t w0 = h ? c.z : c.x, w1 = h ? c.w : c.y;
  return make_uint4(fp8x2_to<DT>(w0), fp8x2_to<DT>(w0 >> 16), fp8x2_to<DT>(w1),
                    fp8x2_to<DT>(w1 >> 16));
}

// the float32 value of a 16-bit element held in a short
template <int DT> __device__ inline float elem_value(short h);
template <> __device__ inline float elem_value<PA_BF16>(short h) {
  return __uint_as_float(uint32_t(static_cast<uint16_t>(h)) << 16);
}
template <> __device__ inline float elem_value<PA_F16>(short h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <int DT, int D, int G>
struct MfmaPv {
  using GE = Geo<DT, D, G>;
  static constexpr int KK = GE::KK, VS = GE::VS, RPI = GE::RPI, CPR = GE::CPR;
  static constexpr int kRowBytes = GE::kRowBytes;
  static constexpr int NT = D / 16;                       // 16-row output tiles of O^T
  static constexpr int kRowsPer256 = 256 / kRowBytes;     // rows sharing one bank sweep
  static constexpr int kScratchBytes = kTileTokens * kRowBytes;   // the wave's V tile
  static_assert(G <= 16, "at most 16 query heads per kv head");

  uint4 qb[KK];
  f32x4 o[NT];
  float m_run, l_run;
  int gq, c, rho, chi;

  __device__ static int swz(int t) { return (2 * (t / kRowsPer256)) & (CPR - 1); }

  __device__ __forceinline__ void set_lane(int lane) {
    gq = lane >> 4;
    c = lane & 15;
    rho = lane / CPR;
    chi = lane % CPR;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = -INFINITY;
    l_run = 0.0f;
  }

  // query rows of the pair from global memory ([G][D] contiguous at qrows)
  __device__ __forceinline__ void init(const DecodeArgs& a, int seq, int g, int lane) {
    set_lane(lane);
    const int head = c < G ? c : G - 1;          // padding columns never dereference
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) +
        (int64_t(seq) * a.num_q_heads + int64_t(g) * G + head) * kRowBytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb[kk] = c < G ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
    reset();
  }

  // query rows of the pair from an LDS copy ([G][D])
  __device__ __forceinline__ void load_q_lds(const char* qs) {
    const int head = c < G ? c : 0;
    const uint4* qrow = reinterpret_cast<const uint4*>(qs + head * kRowBytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb[kk] = c < G ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
  }

  // FP8 pools: key chunk kk of a lane holds elements 16 (gq + 4 kk) .. +16,
  // converted to two MFMA chunks (h = 0, 1); the query chunks follow suit
  __device__ __forceinline__ void load_q_lds_fp8(const char* qs) {
    const int head = c < G ? c : 0;
    const uint4* qrow = reinterpret_cast<const uint4*>(qs + head * kRowBytes);
#pragma unroll
    for (int kk = 0; kk < KK / 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        qb[2 * kk + h] = c < G ? qrow[2 * (gq + 4 * kk) + h] : make_uint4(0, 0, 0, 0);
  }

  float p_[4];
  float alpha_;

  // phase 1: the value tile goes to LDS (chunks swizzled per row)
  __device__ __forceinline__ void stage_values(const ValRegs<DT, D>& r, char* vt) {
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const int row = s * RPI + rho;
      *reinterpret_cast<uint4*>(vt + row * kRowBytes + ((chi ^ swz(row)) << 4)) = r.v[s];
    }
  }

  // phase 2: S^T = K . Q^T, rows >= live masked, online softmax update
  // rows first .. live-1 of the tile take part; the others get weight zero
  __device__ __forceinline__ void scores(const DecodeArgs& a, const KeyRegs<DT, D>& r, int first,
                                         int live) {
    f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sc = mfma_chunk<DT>(r.k[kk], qb[kk], sc);
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      s[i] = row >= first && row < live ? sc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = column_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    alpha_ = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p_[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
      psum += p_[i];
    }
    l_run = fmaf(l_run, alpha_, psum);
    m_run = m_new;
  }

  // phase 3: O^T = alpha O^T + V^T . P^T.  P enters the matrix cores as two
  // element-type operands, hi = P rounded and lo = (P - hi) rounded, so the
  // products carry P to about twice the element type's precision (P rounded
  // once would cost up to half an ulp of the element type per weight; the
  // sum l is taken on the float32 P)
  __device__ __forceinline__ void accumulate(const char* vt) {
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] *= alpha_;
    const v4i16 pb = pack4<DT>(p_);
    float rest[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rest[i] = p_[i] - elem_value<DT>(pb[i]);
    const v4i16 pl = pack4<DT>(rest);
    wave_sync_lds();
    // A operand of tile n: lane (gq, r) points at V[4gq + r/4][16n + 4(r%4)]
    const int row = 4 * gq + (c >> 2);
    const char* rbase = vt + row * kRowBytes + ((c & 1) << 3);
    const int sw = swz(row);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int chunk = 2 * n + ((c & 3) >> 1);
      const v4i16 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(rbase + ((chunk ^ sw) << 4)));
      o[n] = mfma_pv<DT>(av, pb, o[n]);
      o[n] = mfma_pv<DT>(av, pl, o[n]);
    }
    wave_sync_lds();
  }

  // the sum of a head's weights (its four lanes), on every lane
  __device__ __forceinline__ float head_sum() const { return column_sum(l_run); }

  // Compact copy of a piece (O / l times out_scale, and the max and sum per
  // head) for storing later.  Only the first G of the 16 head columns hold
  // results, so the copy spreads them over the other columns' lanes: lane
  // (gq, c) keeps head c % kStashHeads, output tiles b * kStashN + j
  // (j < kStashN) with b = c / kStashHeads, and the max and sum of its head.
  static constexpr int kStashF = G <= 4 ? 4 : G <= 8 ? 2 : 1;
  static constexpr int kStashHeads = 16 / kStashF;
  static constexpr int kStashN = NT / kStashF;
  __device__ __forceinline__ void stash(f32x4* dst, float& m_out, float& l_out, float out_scale) {
    const float l = head_sum();
    const float inv = (1.0f / l) * out_scale;
    const int b = c / kStashHeads;
    const int src = (gq << 4) | (c % kStashHeads);
#pragma unroll
    for (int j = 0; j < kStashN; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int b2 = 0; b2 < kStashF; ++b2) {
          const float t = __shfl(o[b2 * kStashN + j][i] * inv, src, kWave);
          v = b == b2 ? t : v;
        }
        dst[j][i] = v;
      }
    m_out = __shfl(m_run, src, kWave);
    l_out = __shfl(l, src, kWave);
  }
  // store a compact copy to piece slot `piece` of the workspace
  __device__ __forceinline__ void store_stash(const DecodeArgs& a, int piece, const f32x4* st,
                                              float m, float l) {
    const int head = c % kStashHeads;
    if (head >= G) return;
    const int b = c / kStashHeads;
    float* po = a.ws_o + (int64_t(piece) * G + head) * D;
#pragma unroll
    for (int j = 0; j < kStashN; ++j)
      *reinterpret_cast<f32x4*>(po + 16 * (b * kStashN + j) + 4 * gq) = st[j];
    if (gq == 0 && b == 0) {
      a.ws_ml[(piece * G + head) * 2] = m;
      a.ws_ml[(piece * G + head) * 2 + 1] = l;
    }
  }

  // O / l times out_scale, rounded to the element type, into a [G][D] LDS
  // copy of the group's output rows (lane (gq, c < G): d = 16n + 4gq + i)
  __device__ __forceinline__ void stage_output(char* dst, float out_scale) {
    const float l = head_sum();
    if (c >= G) return;
    const float inv = (1.0f / l) * out_scale;
#pragma unroll
    for (int n = 0; n < NT; ++n) store4<DT>(dst, c * D + 16 * n + 4 * gq, o[n] * inv);
  }

  // wave totals into sm: O^T lane (gq, c), element i of tile n = head c, d = 16n + 4gq + i
  template <typename Smem>
  __device__ __forceinline__ void finish(Smem& sm, int wave) {
    float l = l_run;
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (c < G) {
      if (gq == 0) {
        sm.m[wave][c] = m_run;
        sm.l[wave][c] = l;
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.o[wave][c][16 * n + 4 * gq + i] = o[n][i];
    }
  }
};

// ---------------------------------------------------------------------------
// Tile math for float32 elements: QK^T on the float32 matrix cores with the
// query heads repeated down the 16 rows (lane (gq, c) gets token c's scores
// for four heads), softmax reductions across the 16 token lanes by DPP, and
// P.V on the vector ALUs: lane (rho, chi) accumulates chunk chi of its value
// rows for every head, reading the probabilities from a per-wave LDS tile.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
struct ValuPv {
  using GE = Geo<DT, D, G>;
  static constexpr int EPC = GE::EPC, KK = GE::KK, VS = GE::VS, RPI = GE::RPI, CPR = GE::CPR;
  static constexpr int NHB = GE::NHB, kRowBytes = GE::kRowBytes;
  static constexpr int kScratchBytes = kTileTokens * NHB * 16;   // probabilities

  uint4 qa[NHB][KK];
  float m_run[NHB][4], l_run[NHB][4];
  float acc[G][EPC];
  int gq, c, rho, chi;

  __device__ void init(const DecodeArgs& a, int seq, int g, int lane) {
    gq = lane >> 4;
    c = lane & 15;
    rho = lane / CPR;
    chi = lane % CPR;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = 4 * hb + (c & 3);
      const int head_ld = head < G ? head : G - 1;
      const uint4* qrow = reinterpret_cast<const uint4*>(
          static_cast<const char*>(a.q) +
          (int64_t(seq) * a.num_q_heads + int64_t(g) * G + head_ld) * kRowBytes);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qa[hb][kk] = head < G ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m_run[hb][i] = -INFINITY;
        l_run[hb][i] = 0.0f;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;
  }

  ValRegs<DT, D> vals_;
  float pr_[NHB][4];
  f32x4* sp_ = nullptr;

  __device__ void stage_values(const ValRegs<DT, D>& r, char*) { vals_ = r; }

  __device__ void scores(const DecodeArgs& a, const KeyRegs<DT, D>& r, int first, int live) {
    const bool valid = c >= first && c < live;
    float alpha[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = mfma_chunk<DT>(qa[hb][kk], r.k[kk], sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = valid ? sc[i] * a.scale_log2 : -INFINITY;
        const float m_new = fmaxf(m_run[hb][i], row_max16(s));
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        alpha[hb][i] = __builtin_amdgcn_exp2f(m_run[hb][i] - m_use);
        pr_[hb][i] = __builtin_amdgcn_exp2f(s - m_use);
        l_run[hb][i] = l_run[hb][i] * alpha[hb][i] + pr_[hb][i];
        m_run[hb][i] = m_new;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h / 4][h % 4];
  }

  __device__ void accumulate(char* scratch) {
    f32x4* sp = reinterpret_cast<f32x4*>(scratch);        // [16 tokens][NHB]
    if (gq == 0) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        sp[c * NHB + hb] = f32x4{pr_[hb][0], pr_[hb][1], pr_[hb][2], pr_[hb][3]};
    }
    wave_sync_lds();
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      float v[EPC];
      unpack<DT>(vals_.v[s], v);
      const int row = s * RPI + rho;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4 pp = sp[row * NHB + hb];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * hb + i;
          if (h < G) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(pp[i], v[e], acc[h][e]);
          }
        }
      }
    }
    wave_sync_lds();
  }

  template <typename Smem>
  __device__ void finish(Smem& sm, int wave) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[hb][i] = row_sum16(l_run[hb][i]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float x = acc[h][e];
#pragma unroll
        for (int w = CPR; w < kWave; w <<= 1) x += __shfl_xor(x, w, kWave);
        acc[h][e] = x;
      }
    if (gq == 0 && c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sm.m[wave][h] = m_run[h / 4][h % 4];
        sm.l[wave][h] = l_run[h / 4][h % 4];
      }
    }
    if (rho == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm.o[wave][h][chi * EPC + e] = acc[h][e];
    }
  }
};

template <int DT, int D, int G>
struct TileMathFor {
  using type = MfmaPv<DT, D, G>;
};
template <int D, int G>
struct TileMathFor<PA_F32, D, G> {
  using type = ValuPv<PA_F32, D, G>;
};

template <int DT, int D, int G, int NW>
struct SegmentSmem {
  static constexpr int kScratch = TileMathFor<DT, D, G>::type::kScratchBytes;
  alignas(16) char scratch[NW][kScratch];
  float m[NW][G];
  float l[NW][G];
  float o[NW][G][D];
};

// Attend over tiles [tile_lo, tile_hi) (at least one) of pair (seq, g) whose
// sequence holds T > 0 tokens.  Ends with a workgroup barrier after which
// sm.m / sm.l / sm.o hold every wave's max, sum and unnormalised output.
template <int DT, int D, int G, bool kTileInBlock, int NW>
__device__ void attend_segment(const DecodeArgs& a, SegmentSmem<DT, D, G, NW>& sm, int seq, int g,
                               int T, int s0, int tile_lo, int tile_hi) {
  // the segment is the same for every lane; say so, so that addresses and
  // buffer descriptors derived from it stay in scalar registers
  seq = __builtin_amdgcn_readfirstlane(seq);
  g = __builtin_amdgcn_readfirstlane(g);
  T = __builtin_amdgcn_readfirstlane(T);
  s0 = __builtin_amdgcn_readfirstlane(s0);
  tile_lo = __builtin_amdgcn_readfirstlane(tile_lo);
  tile_hi = __builtin_amdgcn_readfirstlane(tile_hi);
  using GE = Geo<DT, D, G>;
  constexpr int KK = GE::KK, RPI = GE::RPI, VS = GE::VS, CPR = GE::CPR;
  constexpr int kRowBytes = GE::kRowBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gq = lane >> 4;
  const int c = lane & 15;
  const int rho = lane / CPR;
  const int chi = lane % CPR;

  typename TileMathFor<DT, D, G>::type tm;
  tm.init(a, seq, g, lane);

  const int lb = a.log2_block;
  const int bmask = (1 << lb) - 1;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq;
  const int64_t head_rows = int64_t(g) << lb;                 // kv head g inside a block
  const int64_t blk_rows = int64_t(a.num_kv_heads) << lb;     // rows per block
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int nblk = a.num_blocks;

  const int span = tile_hi - tile_lo - wave;
  const int nmine = span > 0 ? (span + NW - 1) / NW : 0;

  // block ids of this wave's tiles, 64 tiles per load: lane j holds the block
  // of the wave's tile 64*batch + j (used when a tile lies inside one block)
  int tbl = 0;
  auto load_tbl = [&](int batch) {
    const int k = min(64 * batch + lane, nmine - 1);
    const int t = min((tile_lo + wave + NW * k) * kTileTokens, T - 1);
    tbl = min(max(table[t >> lb], 0), nblk - 1);
  };

  // per-lane byte offsets inside a tile's 16 rows (constant for the segment)
  const int k_off = c * kRowBytes + gq * 16;          // key chunk gq of row c; +64 per kk
  const int v_off = rho * kRowBytes + chi * 16;       // value chunk chi of row rho
  auto tile_start = [&](int kidx) { return (tile_lo + wave + NW * kidx) * kTileTokens; };
  auto tile_byte = [&](int kidx, int t0) -> int64_t {
    const int64_t blk = __builtin_amdgcn_readlane(tbl, kidx & 63);
    return (blk * blk_rows + head_rows + (t0 & bmask)) * kRowBytes;
  };
  // The tile's 16 rows are contiguous inside one (block, kv head) run: a
  // buffer descriptor spans exactly the live rows, so rows past T-1 (the tail
  // of the sequence's last tile) load as zeros and are never read.
  auto rsrc = [&](const char* base, int64_t byte, int t0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + byte), 0,
                                             min(kTileTokens, T - t0) * kRowBytes, kBufferDword3);
  };
  // Without that (blocks smaller than a tile) each lane finds its own block;
  // tokens past T-1 read row T-1 and tokens before the window's first
  // position s0 read row s0 (data of this sequence, weight zero), so no table
  // entry outside the attended positions is read.
  auto row_of = [&](int t0, int dt) -> int64_t {
    const int t = max(s0, t0 + min(dt, T - 1 - t0));
    const int64_t blk = min(max(table[t >> lb], 0), nblk - 1);
    return blk * blk_rows + head_rows + (t & bmask);
  };
  auto load_keys = [&](int kidx, KeyRegs<DT, D>& r) {
    const int t0 = tile_start(kidx);
    if constexpr (kTileInBlock) {
      const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, tile_byte(kidx, t0), t0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        r.k[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + 64 * kk, 0, 0));
    } else {
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + row_of(t0, c) * kRowBytes);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) r.k[kk] = kp[4 * kk + gq];
    }
  };
  auto load_values = [&](int kidx, ValRegs<DT, D>& r) {
    const int t0 = tile_start(kidx);
    if constexpr (kTileInBlock) {
      const __amdgpu_buffer_rsrc_t rv = rsrc(vbase, tile_byte(kidx, t0), t0);
#pragma unroll
      for (int s = 0; s < VS; ++s)
        r.v[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rv, v_off + s * RPI * kRowBytes, 0, 0));
    } else {
#pragma unroll
      for (int s = 0; s < VS; ++s)
        r.v[s] = reinterpret_cast<const uint4*>(vbase + row_of(t0, s * RPI + rho) * kRowBytes)[chi];
    }
  };

  char* scratch = sm.scratch[wave];
  // Keys are double-buffered in registers; values are single-buffered: the
  // next tile's values are requested as soon as this tile's are in LDS.
  if (nmine > 0) {
    if constexpr (kTileInBlock) load_tbl(0);
    KeyRegs<DT, D> KA, KB;
    ValRegs<DT, D> VR;
    load_keys(0, KA);
    load_values(0, VR);
    if (nmine > 1) load_keys(1, KB);
    auto step = [&](int k, KeyRegs<DT, D>& kr) {
      const int t0 = tile_start(k);
      const int first = max(0, s0 - t0);
      if (first > 0) clear_rows_below(VR, first, rho);
      tm.stage_values(VR, scratch);
      if (k + 1 < nmine) load_values(k + 1, VR);
      tm.scores(a, kr, first, min(kTileTokens, T - t0));
      if (k + 2 < nmine) {
        if (kTileInBlock && ((k + 2) & 63) == 0) load_tbl((k + 2) >> 6);
        load_keys(k + 2, kr);
      }
      tm.accumulate(scratch);
    };
    for (int k = 0; k < nmine; k += 2) {
      step(k, KA);
      if (k + 1 >= nmine) break;
      step(k + 1, KB);
    }
  }
  // a wave without tiles reports m = -inf, l = 0, o = 0
  tm.finish(sm, wave);
  __syncthreads();
}

// Merge the four waves' results for (head h, element d): M = max, L = sum of
// 2^(m_w - M) l_w, O = sum of 2^(m_w - M) o_w.  The attention output is O / L.
template <int DT, int D, int G, int NW>
__device__ inline void merge_waves(const SegmentSmem<DT, D, G, NW>& sm, int h, int d, float& M,
                                   float& L, float& O) {
  M = sm.m[0][h];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
  L = 0.0f;
  O = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float f = __builtin_amdgcn_exp2f(sm.m[w][h] - M);
    L = fmaf(f, sm.l[w][h], L);
    O = fmaf(f, sm.o[w][h][d], O);
  }
}

template <int DT, int D>
__device__ inline void zero_rows(const DecodeArgs& a, int64_t row0, int nrows) {
  for (int i = threadIdx.x; i < nrows * D; i += blockDim.x)
    store_elem<DT>(a.out, row0 * D + i, 0.0f);
}

// ---------------------------------------------------------------------------
// Balanced split (the default for 16-bit elements and blocks of >= 16
// tokens).  The grid holds as many one-wave workgroups as the GPU keeps
// resident.  The flattened work (sequence, kv head, 16-token tile) is cut
// into contiguous shares, one per wave, sized so that long and short
// sequences load every wave alike.
//
// Start of a wave: one round trip brings every length (lane l holds
// sequences l, l + 64, ...); a scan over them gives each sequence's place in
// the flattened work, and the share's segments ((sequence, kv head) pairs or
// parts of them) are found by the lanes in parallel, one candidate sequence
// per lane.  A second round trip brings the block-table entries of the first
// 64 tiles and the segments' query rows, and the first tiles' keys and values
// are requested.  Tiles then stream without draining at segment boundaries:
// keys two tiles ahead, values one tile ahead, the table entries of the next
// 64 tiles half a batch ahead.
//
// Nothing is stored while tiles are in flight (a store counts in the same
// in-order counter as the loads, so every later wait would include it): a
// complete pair's output is staged in LDS over its query rows, the share's
// first segment, when it is a piece of a pair cut by the share's start, is
// kept in registers, and all of it is written after the run's last tile.  A
// pair cut by a share boundary leaves a "piece" (max, sum, normalised output
// per head) in slot 0 (the share's first segment) or slot 1 (its last); the
// first piece also records how many shares the pair spans, and the piece
// merge kernel combines them.
// ---------------------------------------------------------------------------
constexpr int kPieceFirst = 1;   // the piece starts at the pair's first tile
constexpr int kPieceLast = 2;    // the piece ends at the pair's last tile
constexpr int kHdrInts = 8;      // valid, seq, kv head, flags, pieces, (pad)
constexpr int kQStageBytes = 6144;   // LDS for query rows (and new rows) of one run
constexpr int kMetaLive = 0x1f;    // tile descriptor: live rows (1..16)
constexpr int kMetaAppend = 0x20;  // tile descriptor: the last live row is appended
constexpr int kMetaStore = 0x40;   // ... and its table entry lies in the pool

constexpr int kPairCost = 1;

// Cache policy of the key and value loads when the batch streams (the host
// sets DecodeArgs::kv_stream for batches whose KV bytes may exceed the 256 MB
// Infinity Cache): non-temporal (the "nt" bit).  Reads of shuffled 4 KiB
// tiles measured 12% faster so, and the eight XCDs finished together (with
// the default policy the odd XCD of each pair finished about 6% later).
// Smaller batches keep the default policy: blocks that several sequences
// share (a common prefix) are then read from the caches after the first read.
constexpr int kStreamLoad = 2;

__device__ inline int pair_units(int T, int window) {
  const int tiles = attended_tiles(T, window);
  return tiles ? tiles + kPairCost : 0;
}

// first unit of share w of nsh equal shares (total units < 2^31)
__device__ inline int share_lo(int total, int w, int nsh) {
  return static_cast<int>(static_cast<long long>(total) * w / nsh);
}
// the share holding unit u < total: the largest w with share_lo(w) <= u,
// i.e. total * w < (u + 1) * nsh, so w = ceil((u + 1) * nsh / total) - 1
__device__ inline int share_of(int total, int u, int nsh) {
  return static_cast<int>(((static_cast<long long>(u) + 1) * nsh + total - 1) / total) - 1;
}

template <int DT, int D, int G, bool kAppend>
struct StreamSmem {
  static constexpr int kRowBytes = Geo<DT, D, G>::kRowBytes;
  static constexpr int kQBytes = G * D * 2;
  // appending decode: each segment's new K and V rows sit beside its queries
  static constexpr int kNewBytes = kAppend ? 2 * kRowBytes : 0;
  static constexpr int kSegCap = std::max(1, std::min(16, kQStageBytes / (kQBytes + kNewBytes)));
  alignas(16) char vtile[MfmaPv<DT, D, G>::kScratchBytes];
  // a segment's query rows; a complete pair's output rows once it is done
  alignas(16) char q[kSegCap][kQBytes];
  // per sequence: pair units before it (per kv head) and its clamped length
  int2 seq[kMaxSplitSeqs + 1];
  int32_t seg_seq[kSegCap];
  int32_t seg_g[kSegCap];
  int32_t seg_tile0[kSegCap];     // absolute tile index of the segment's first tile
  int32_t seg_start[kSegCap];     // its index in the run's tile list
  int32_t seg_n[kSegCap];
  int32_t seg_T[kSegCap];
  int32_t seg_flags[kSegCap];     // kPieceFirst | kPieceLast, 4: the share's first segment
  int32_t seg_pieces[kSegCap];    // shares the pair spans (pieces that start it)
  int32_t run_end;                // unit after the run's last segment
  int32_t run_seq;                // sequence of the run's last segment
  alignas(16) char newkv[kAppend ? kSegCap : 1][kAppend ? kNewBytes : 16];
  int64_t new_dst[kAppend ? kSegCap : 1];   // pool byte offset of the new row, or -1
};

template <int DT, int D, int G, bool kAppend, bool kWindow, bool kFp8>
__global__ __launch_bounds__(kWave) void decode_stream_kernel(DecodeArgs a) {
  using GE = Geo<DT, D, G>;
  using SM = StreamSmem<DT, D, G, kAppend>;
  using TM = MfmaPv<DT, D, G>;
  const int window = kWindow ? a.window : 0;      // 0: every token
  // pool rows: D codes (FP8 pools) or D elements of DT; the query rows, the LDS
  // value tile and the tile math always use DT
  constexpr int kPoolRowBytes = kFp8 ? D : GE::kRowBytes;
  constexpr int CPR = kPoolRowBytes / 16;         // 16-byte chunks per pool row
  constexpr int KK = CPR / 4;                     // key chunks per lane per tile
  constexpr int RPI = kWave / CPR;                // value rows per load instruction
  constexpr int VS = kTileTokens / RPI;           // value loads per lane per tile
  constexpr int kRowBytes = GE::kRowBytes;
  constexpr int kRows = kMaxSplitSeqs / kWave;
  constexpr int kQChunks = SM::kQBytes / 16;
  __shared__ SM sm;

  const int w = blockIdx.x;
  const int W = gridDim.x;
  const int N = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int lane = threadIdx.x;
  const int nrows = (N + kWave - 1) / kWave;

  // ---- clamped lengths: every load in flight at once, through a buffer
  //      descriptor over the N lengths (a lane past the last sequence reads 0
  //      without touching memory, so no branch separates the loads) ----
  int len[kRows];
  {
    const __amdgpu_buffer_rsrc_t lens = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.context_lens), 0, N * 4, kBufferDword3);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      len[r] = static_cast<int>(
          __builtin_amdgcn_raw_buffer_load_b32(lens, (r * kWave + lane) * 4, 0, 0));
#pragma unroll
    for (int r = 0; r < kRows; ++r) len[r] = min(max(len[r], 0), a.max_context_len);
  }
  // ---- pair units before each sequence: a scan over the lanes, row by row ----
  int pre[kRows];
  int carry = 0;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    pre[r] = 0;
    if (r < nrows) {
      const int u = pair_units(len[r], window);
      const int incl = wave_scan_incl(u);
      pre[r] = carry + incl - u;
      const int s = r * kWave + lane;
      if (s < N) sm.seq[s] = make_int2(pre[r], len[r]);
      carry += wave_last(incl);
    }
  }
  if (lane == 0) sm.seq[N] = make_int2(carry, 0);
  // units: per (sequence, kv head) pair, its tiles plus kPairCost (the fixed
  // cost of a segment: query rows, the partial last tile, the result)
  const int total = Hkv * carry;                  // below 2^31 (the plan checks it)
  const int want = (total + a.min_split_tiles - 1) / a.min_split_tiles;
  const int nsh = max(1, min(W, want));
  const int lo = (w < nsh && total > 0) ? share_lo(total, w, nsh) : 0;
  const int hi = (w < nsh && total > 0) ? share_lo(total, w + 1, nsh) : 0;
  // the share's first sequence: the last s whose work starts at or before lo
  int first_seq = -1;
#pragma unroll
  for (int r = 0; r < kRows; ++r)
    if (r < nrows)
      first_seq += __popcll(__ballot(r * kWave + lane < N && Hkv * pre[r] <= lo));
  wave_sync_lds();

  TM tm;
  tm.set_lane(lane);
  const int gq = lane >> 4, c = lane & 15, rho = lane / CPR, chi = lane % CPR;
  const int k_off = c * kPoolRowBytes + gq * 16;      // key chunk gq of row c; +64 per kk
  const int v_off = rho * kPoolRowBytes + chi * 16;   // value chunk chi of row rho
  const int lb = a.log2_block;
  const int bmask = (1 << lb) - 1;
  const int64_t blk_rows = int64_t(Hkv) << lb;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const float out_scale = kFp8 ? a.v_scale : 1.0f;

  // piece headers of the share (slot 0: its first segment, slot 1: its
  // last), written when the share is done
  // (valid, sequence, kv head, flags, pieces) of each slot
  int h0_valid = 0, h0_seq = 0, h0_g = 0, h0_flags = 0, h0_pieces = 0;
  int h1_valid = 0, h1_seq = 0, h1_g = 0, h1_flags = 0, h1_pieces = 0;
  // the share's first segment when it is a piece and more segments follow:
  // normalised output, max and sum, stored when the share is done
  f32x4 stash_o[TM::kStashN];
  float stash_m = 0.0f, stash_l = 0.0f;
  bool stashed = false;

  int pos = lo;
  int s_cur = max(first_seq, 0);
  while (pos < hi) {
    // ---- the next run of segments: lane j looks at sequence s_cur + j ----
    int nmine = 0, g_first = 0, P = 0, u = 0, T = 0, my_tiles = 0;
    const int s_lane = s_cur + lane;
    if (s_lane < N) {
      const int2 cur = sm.seq[s_lane];
      P = cur.x;
      T = cur.y;
      u = sm.seq[s_lane + 1].x - P;
      const int beg = Hkv * P;
      const int a0 = max(pos, beg), a1 = min(hi, beg + Hkv * u);
      if (u > 0 && a0 < a1) {
        g_first = (a0 - beg) / u;
        int g_last = (a1 - 1 - beg) / u;
        // a pair the share reaches only through its first unit holds none of its tiles
        if (a1 - (beg + g_last * u) <= kPairCost) --g_last;
        nmine = max(0, g_last - g_first + 1);
      }
    }
    // (row shifts and broadcasts on the vector ALU, not a chain of round
    // trips through LDS; the totals are still shuffled from the last lane:
    // read as wave-uniform scalars they change the tile loop's code, which
    // then took 256 registers and ran 3 us longer on the Llama-3-8B batch)
    const int incl = wave_scan_incl(nmine);
    const int seg_before = incl - nmine;
    const int nseg_all = __shfl(incl, kWave - 1, kWave);
    const int nseg = min(nseg_all, SM::kSegCap);
    // tiles of this lane's segments that fit the run
    const int beg = Hkv * P;
    auto seg_tiles = [&](int i, int& t0, int& t1) {
      const int ps = beg + (g_first + i) * u;
      t0 = max(0, pos - ps - kPairCost);
      t1 = min(hi, ps + u) - ps - kPairCost;
    };
    for (int i = 0; i < nmine && seg_before + i < SM::kSegCap; ++i) {
      int t0, t1;
      seg_tiles(i, t0, t1);
      my_tiles += t1 - t0;
    }
    const int tincl = wave_scan_incl(my_tiles);
    const int ntot = __shfl(tincl, kWave - 1, kWave);
    {
      int start = tincl - my_tiles;
      const int wf = window_first(T, window) / kTileTokens;
      for (int i = 0; i < nmine && seg_before + i < SM::kSegCap; ++i) {
        const int slot = seg_before + i;
        const int g = g_first + i;
        int t0, t1;
        seg_tiles(i, t0, t1);
        const int ps = beg + g * u;
        int flags = (t0 == 0 ? kPieceFirst : 0) | (t1 == u - kPairCost ? kPieceLast : 0);
        if (slot == 0 && pos == lo) flags |= 4;
        sm.seg_seq[slot] = s_lane;
        sm.seg_g[slot] = g;
        sm.seg_tile0[slot] = wf + t0;
        sm.seg_start[slot] = start;
        sm.seg_n[slot] = t1 - t0;
        sm.seg_T[slot] = T;
        sm.seg_flags[slot] = flags;
        // a piece that starts its pair: shares up to the one holding its last unit
        sm.seg_pieces[slot] = (flags & 3) == kPieceFirst ? share_of(total, ps + u - 1, nsh) - w + 1 : 1;
        if constexpr (kAppend) sm.new_dst[slot] = -1;
        if (slot == nseg - 1) {
          sm.run_end = ps + kPairCost + t1;
          sm.run_seq = s_lane;
        }
        start += t1 - t0;
      }
    }
    if (nseg == 0) {
      // no tile of [pos, hi) among these 64 sequences (they are empty, or the
      // share ends on a pair's tile-less first unit): move past them
      const int s_next = s_cur + kWave;
      if (s_next >= N) break;
      pos = max(pos, Hkv * sm.seq[s_next].x);
      s_cur = s_next;
      continue;
    }
    wave_sync_lds();
    const int run_end = nseg_all > nseg ? sm.run_end
                                        : min(hi, s_cur + kWave < N ? Hkv * sm.seq[s_cur + kWave].x : hi);
    const int run_seq = sm.run_seq;
    const bool share_done = run_end >= hi;

    // ---- per-tile descriptors, 64 tiles per batch: lane j holds tile
    //      64*batch + j: its first row's byte offset and (segment, live rows)
    auto tile_seg = [&](int j) {
      int sg = 0;
      for (int i = 1; i < nseg; ++i)
        if (j >= sm.seg_start[i]) sg = i;
      return sg;
    };
    auto table_entry = [&](int j, int& sg, int& t0) {
      sg = tile_seg(j);
      t0 = (sm.seg_tile0[sg] + j - sm.seg_start[sg]) * kTileTokens;
      const int32_t* table = a.block_tables + int64_t(sm.seg_seq[sg]) * a.max_blocks_per_seq;
      return table[min(max(t0, 0) >> lb, a.max_blocks_per_seq - 1)];   // (always in range)
    };
    int64_t doff = 0;
    int dmeta = 0;
    auto make_desc = [&](int32_t entry, int sg, int t0) {
      const int Ts = sm.seg_T[sg];
      const int64_t blk = min(max(entry, 0), a.num_blocks - 1);
      doff = (blk * blk_rows + (int64_t(sm.seg_g[sg]) << lb) + (t0 & bmask)) * kPoolRowBytes;
      const int live = min(kTileTokens, Ts - t0);
      // the sequence's newest token is in this tile and comes from new_k/new_v
      const bool app = kAppend && t0 + live == Ts;
      const bool in_pool = entry == blk;
      const int first = kWindow ? max(0, window_first(Ts, window) - t0) : 0;   // rows before it
      dmeta = live | (app ? kMetaAppend : 0) | (app && in_pool ? kMetaStore : 0) | (sg << 8) |
              (first << 12);
    };
    int nx_entry = 0, nx_sg = 0, nx_t0 = 0;     // table entry of the next batch (prefetched)

    auto tile_off = [&](int k) -> int64_t {
      const uint32_t lo32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(doff), k & 63);
      const uint32_t hi32 = __builtin_amdgcn_readlane(static_cast<uint32_t>(doff >> 32), k & 63);
      return (int64_t(hi32) << 32) | lo32;
    };
    auto tile_meta = [&](int k) -> int { return __builtin_amdgcn_readlane(dmeta, k & 63); };
    // A tile's rows are contiguous in one (block, kv head) run.  The buffer
    // descriptor starts at the first attended row (the window's first
    // position in its tile, else row 0) and stops after the last row the
    // pool supplies, so rows past a sequence's end, and rows before a
    // window, read as zeros without touching memory: their lane offsets fall
    // outside the descriptor (below its start they wrap around as unsigned
    // offsets).
    auto rsrc = [&](const char* base, int64_t off, int first, int rows) {
      return __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(base + off + first * kPoolRowBytes), 0,
          max(0, rows - first) * kPoolRowBytes, kBufferDword3);
    };
    struct Keys {
      KeyRegs<DT, D> r;
      int meta;
      int64_t off;                   // byte offset of the tile's first row in the pools
    };
    // rows the pool supplies: the live ones, less the newest when it is
    // appended (that row then reads as zero and never touches the pool)
    auto pool_rows = [&](int meta) {
      return (meta & kMetaLive) - ((kAppend && (meta & kMetaAppend)) ? 1 : 0);
    };
    auto first_row = [&](int meta) { return kWindow ? (meta >> 12) & 0xf : 0; };
    auto load_keys = [&](int k, Keys& kr) {
      if ((k & 63) == 0 && k > 0) make_desc(nx_entry, nx_sg, nx_t0);
      const int meta = tile_meta(k);
      const int64_t off = tile_off(k);
      const int first = first_row(meta);
      const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, off, first, pool_rows(meta));
      const int shift = first * kPoolRowBytes;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kr.r.k[kk] = __builtin_bit_cast(
            uint4, a.kv_stream ? __builtin_amdgcn_raw_buffer_load_b128(
                                     rk, k_off + 64 * kk - shift, 0, kStreamLoad)
                               : __builtin_amdgcn_raw_buffer_load_b128(
                                     rk, k_off + 64 * kk - shift, 0, 0));
      kr.meta = meta;
      kr.off = off;
    };
    ValRegs<DT, D> vr;
    auto load_vals = [&](int k) {
      const int meta = tile_meta(k);
      const int first = first_row(meta);
      const __amdgpu_buffer_rsrc_t rv = rsrc(vbase, tile_off(k), first, pool_rows(meta));
      const int shift = first * kPoolRowBytes;
#pragma unroll
      for (int s2 = 0; s2 < VS; ++s2)
        vr.v[s2] = __builtin_bit_cast(
            uint4, a.kv_stream ? __builtin_amdgcn_raw_buffer_load_b128(
                                     rv, v_off + s2 * RPI * kPoolRowBytes - shift, 0, kStreamLoad)
                               : __builtin_amdgcn_raw_buffer_load_b128(
                                     rv, v_off + s2 * RPI * kPoolRowBytes - shift, 0, 0));
    };
    // Appending tile: the newest row of the keys and of the values comes from
    // the segment's LDS copy of new_k / new_v (register selects only, so the
    // loads in flight are not waited for any earlier than the tile needs).
    // This wave, the only one to handle that row, also stores it to its pool
    // slot once the run's tiles are done.  Nothing reads that slot in this
    // launch: the descriptors of the tile stop short of it.
    auto put_new_row = [&](Keys& kr) {
      const int live = kr.meta & kMetaLive;
      const char* nk = sm.newkv[(kr.meta >> 8) & 0xf];
      if (lane == 0)
        sm.new_dst[(kr.meta >> 8) & 0xf] =
            (kr.meta & kMetaStore) ? kr.off + int64_t(live - 1) * kPoolRowBytes : int64_t(-1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 x = *reinterpret_cast<const uint4*>(nk + (gq + 4 * kk) * 16);
        if (c == live - 1) kr.r.k[kk] = x;
      }
      const uint4 y = *reinterpret_cast<const uint4*>(nk + kPoolRowBytes + chi * 16);
#pragma unroll
      for (int s2 = 0; s2 < VS; ++s2)
        if (rho + s2 * RPI == live - 1) vr.v[s2] = y;
    };

    // ---- second round trip: the first batch's table entries, then the
    //      segments' query rows and new rows; the first tiles' keys and
    //      values are requested before any of the rows is waited for ----
    Keys KA, KB;
    {
      int sg0, t00;
      const int32_t entry0 = table_entry(min(lane, ntot - 1), sg0, t00);
      // (every lane loads: chunks past the run's last one repeat it, so the
      // loads need no branches and stay in registers until written to LDS)
      constexpr int kQPerLane = (SM::kSegCap * kQChunks + kWave - 1) / kWave;
      uint4 qv[kQPerLane];
#pragma unroll
      for (int i = 0; i < kQPerLane; ++i) {
        const int idx = min(lane + i * kWave, nseg * kQChunks - 1);
        const int sgq = idx / kQChunks;
        qv[i] = reinterpret_cast<const uint4*>(
            static_cast<const char*>(a.q) +
            (int64_t(sm.seg_seq[sgq]) * Hq + int64_t(sm.seg_g[sgq]) * G) *
                kRowBytes)[idx - sgq * kQChunks];
      }
      // appending decode: each segment's new K row, then its new V row
      // (16-bit elements: 2 * kRowBytes / 16 chunks per segment)
      constexpr int kNewChunks = 2 * kRowBytes / 16;
      constexpr int kNPerLane = kAppend ? (SM::kSegCap * kNewChunks + kWave - 1) / kWave : 1;
      uint4 nv[kNPerLane];
      if constexpr (kAppend) {
#pragma unroll
        for (int i = 0; i < kNPerLane; ++i) {
          const int idx = min(lane + i * kWave, nseg * kNewChunks - 1);
          const int sgn = idx / kNewChunks;
          const int part = idx - sgn * kNewChunks;
          const bool is_v = part >= kNewChunks / 2;
          nv[i] = reinterpret_cast<const uint4*>(
              static_cast<const char*>(is_v ? a.new_v : a.new_k) +
              (int64_t(sm.seg_seq[sgn]) * Hkv + sm.seg_g[sgn]) *
                  kRowBytes)[is_v ? part - kNewChunks / 2 : part];
        }
      }
      make_desc(entry0, sg0, t00);
      load_keys(0, KA);
      load_vals(0);
      if (ntot > 1) load_keys(1, KB);
#pragma unroll
      for (int i = 0; i < kQPerLane; ++i) {
        const int idx = lane + i * kWave;
        if (idx < nseg * kQChunks) {
          const int sgq = idx / kQChunks;
          *reinterpret_cast<uint4*>(sm.q[sgq] + (idx - sgq * kQChunks) * 16) = qv[i];
        }
      }
      if constexpr (kAppend) {
#pragma unroll
        for (int i = 0; i < kNPerLane; ++i) {
          const int idx = lane + i * kWave;
          if (idx < nseg * kNewChunks) {
            const int sgn = idx / kNewChunks;
            const int part = idx - sgn * kNewChunks;
            if constexpr (kFp8) {
              // FP8 pools: the new rows are quantized as the FP8 slot write
              // does (the codes of x / scale) and kept as codes, which then
              // take the pool rows' path through the tile math and are the
              // bytes stored to the slot: 8 elements -> 8 codes per chunk
              const bool is_v = part >= kNewChunks / 2;
              const int ch = is_v ? part - kNewChunks / 2 : part;
              const float sc = is_v ? a.v_scale : a.k_scale;
              const uint4 x = nv[i];
              const uint32_t hw[8] = {x.x & 0xffffu, x.x >> 16, x.y & 0xffffu, x.y >> 16,
                                      x.z & 0xffffu, x.z >> 16, x.w & 0xffffu, x.w >> 16};
              float y[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = half_bits_to_float<DT>(hw[e]) / sc;
              const uint2 codes = make_uint2(e4m3_codes4(y[0], y[1], y[2], y[3]),
                                             e4m3_codes4(y[4], y[5], y[6], y[7]));
              *reinterpret_cast<uint2*>(sm.newkv[sgn] + (is_v ? kPoolRowBytes : 0) + 8 * ch) =
                  codes;
            } else {
              *reinterpret_cast<uint4*>(sm.newkv[sgn] + part * 16) = nv[i];
            }
          }
        }
      }
    }
    wave_sync_lds();                 // the query rows (and new rows) are in LDS
    int cur = -1;
    int last_sg = -1;                // the run's last segment when it is a piece left in registers
    auto step = [&](int k, Keys& kr) {
      const int sg = (kr.meta >> 8) & 0xf;
      if (sg != cur) {               // a new segment begins
        cur = sg;
        tm.reset();
        if constexpr (kFp8)
          tm.load_q_lds_fp8(sm.q[sg]);
        else
          tm.load_q_lds(sm.q[sg]);
      }
      // the next batch's table entries, half a batch ahead
      if ((k & 63) == 32 && (k | 63) + 1 < ntot)
        nx_entry = table_entry(min((k | 63) + 1 + lane, ntot - 1), nx_sg, nx_t0);
      if constexpr (kAppend)
        if (kr.meta & kMetaAppend) put_new_row(kr);
      const int first = first_row(kr.meta);
      if constexpr (kFp8) {
        // each chunk of 16 value codes becomes two 16-bit chunks of the row
#pragma unroll
        for (int s2 = 0; s2 < VS; ++s2) {
          const int row = s2 * RPI + rho;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<uint4*>(sm.vtile + row * kRowBytes +
                                      (((2 * chi + h) ^ TM::swz(row)) << 4)) =
                fp8x8_to<DT>(vr.v[s2], h);
        }
      } else {
        tm.stage_values(vr, sm.vtile);
      }
      if (k + 1 < ntot) load_vals(k + 1);
      if constexpr (kFp8) {
        KeyRegs<DT, D> kb;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kb.k[2 * kk] = fp8x8_to<DT>(kr.r.k[kk], 0);
          kb.k[2 * kk + 1] = fp8x8_to<DT>(kr.r.k[kk], 1);
        }
        tm.scores(a, kb, first, kr.meta & kMetaLive);
      } else {
        tm.scores(a, kr.r, first, kr.meta & kMetaLive);
      }
      if (k + 2 < ntot) load_keys(k + 2, kr);
      tm.accumulate(sm.vtile);
      if (k + 1 == sm.seg_start[sg] + sm.seg_n[sg]) {   // the segment's last tile
        const int flags = sm.seg_flags[sg];
        if ((flags & 3) == (kPieceFirst | kPieceLast)) {
          tm.stage_output(sm.q[sg], out_scale);          // over its (spent) query rows
        } else if ((flags & 4) && !(share_done && k + 1 == ntot)) {
          // the share's first segment, a piece, with more segments to come
          tm.stash(stash_o, stash_m, stash_l, out_scale);
          stashed = true;
          h0_valid = 1;
          h0_seq = sm.seg_seq[sg];
          h0_g = sm.seg_g[sg];
          h0_flags = flags & 3;
          h0_pieces = sm.seg_pieces[sg];
        } else {
          last_sg = sg;              // the share's last segment: stored after the loop
        }
      }
    };
    for (int k = 0; k < ntot; k += 2) {
      step(k, KA);
      if (k + 1 >= ntot) break;
      step(k + 1, KB);
    }

    // ---- the run is done: results and appended rows leave the wave ----
    if (last_sg >= 0) {
      const int flags = sm.seg_flags[last_sg];
      const int slot = (flags & 4) ? 0 : 1;
      const int piece = 2 * w + slot;
      const float l = tm.head_sum();
      if (c < G) {
        const float inv = (1.0f / l) * out_scale;
        float* po = a.ws_o + (int64_t(piece) * G + c) * D;
#pragma unroll
        for (int n = 0; n < TM::NT; ++n)
          *reinterpret_cast<f32x4*>(po + 16 * n + 4 * gq) = tm.o[n] * inv;
        if (gq == 0) {
          a.ws_ml[(piece * G + c) * 2] = tm.m_run;
          a.ws_ml[(piece * G + c) * 2 + 1] = l;
        }
      }
      if (slot == 0) {
        h0_valid = 1;
        h0_seq = sm.seg_seq[last_sg];
        h0_g = sm.seg_g[last_sg];
        h0_flags = flags & 3;
        h0_pieces = sm.seg_pieces[last_sg];
      } else {
        h1_valid = 1;
        h1_seq = sm.seg_seq[last_sg];
        h1_g = sm.seg_g[last_sg];
        h1_flags = flags & 3;
        h1_pieces = sm.seg_pieces[last_sg];
      }
    }
    wave_sync_lds();                 // staged outputs and new_dst records
    for (int idx = lane; idx < nseg * kQChunks; idx += kWave) {
      const int sg = idx / kQChunks;
      if ((sm.seg_flags[sg] & 3) != (kPieceFirst | kPieceLast)) continue;
      const int part = idx - sg * kQChunks;
      reinterpret_cast<uint4*>(static_cast<char*>(a.out) +
                               (int64_t(sm.seg_seq[sg]) * Hq + int64_t(sm.seg_g[sg]) * G) *
                                   kRowBytes)[part] =
          *reinterpret_cast<const uint4*>(sm.q[sg] + part * 16);
    }
    if constexpr (kAppend) {
      for (int sg = 0; sg < nseg; ++sg) {
        const int64_t dst = sm.new_dst[sg];
        if (dst >= 0 && lane < 2 * CPR) {
          const bool is_v = lane >= CPR;
          char* pool = const_cast<char*>(is_v ? vbase : kbase);
          *reinterpret_cast<uint4*>(pool + dst + (is_v ? lane - CPR : lane) * 16) =
              *reinterpret_cast<const uint4*>(sm.newkv[sg] + lane * 16);
        }
      }
    }
    wave_sync_lds();                 // LDS records are rewritten by the next run
    pos = run_end;
    s_cur = nseg_all > nseg ? run_seq : min(N, s_cur + kWave);
  }

  // ---- the share is done ----
  if (stashed) tm.store_stash(a, 2 * w, stash_o, stash_m, stash_l);
  if (lane < 2) {
    int32_t* hdr = a.ws_hdr + (2 * w + lane) * kHdrInts;
    hdr[0] = lane ? h1_valid : h0_valid;
    hdr[1] = lane ? h1_seq : h0_seq;
    hdr[2] = lane ? h1_g : h0_g;
    hdr[3] = lane ? h1_flags : h0_flags;
    hdr[4] = lane ? h1_pieces : h0_pieces;
  }
  // zero-length sequences get zero rows (spread over every workgroup)
  for (int s = w; s < N; s += W)
    if (sm.seq[s].y == 0) zero_rows<DT, D>(a, int64_t(s) * Hq, Hq);
}

// Combine the pieces of every pair that starts inside this share: the piece
// here (slot 0 or 1) and slot 0 of the next pieces-1 shares.  One workgroup
// per share, one thread per float4 quad of the pair's [G][D] output (so that
// every load of a batch is in flight at once).  Both headers and, in the same
// round trip, the two pieces a pair starting here most often has (this
// share's slot 1, the next share's slot 0) are loaded together; further
// pieces follow kBatch at a time.  The fold order is fixed by the split alone,
// so results do not depend on timing.
template <int G, int D>
struct MergeShape {
  static constexpr int kQuads = G * D / 4;
  static constexpr int kThreads = std::min(256, (kQuads + kWave - 1) / kWave * kWave);
  static constexpr int kQPT = (kQuads + kThreads - 1) / kThreads;   // quads per thread
};

template <int DT, int D, int G>
__global__ __launch_bounds__((MergeShape<G, D>::kThreads)) void merge_pieces_kernel(DecodeArgs a,
                                                                                    int W) {
  using MS = MergeShape<G, D>;
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  constexpr int kQuads = MS::kQuads;
  constexpr int kQPT = MS::kQPT;
  constexpr int kBatch = 8;
  int hvalid[2], hseq[2], hg[2], hflags[2], hnp[2];
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    const int32_t* hdr = a.ws_hdr + (2 * w + slot) * kHdrInts;
    hvalid[slot] = __builtin_amdgcn_readfirstlane(hdr[0]);
    hseq[slot] = __builtin_amdgcn_readfirstlane(hdr[1]);
    hg[slot] = __builtin_amdgcn_readfirstlane(hdr[2]);
    hflags[slot] = __builtin_amdgcn_readfirstlane(hdr[3]);
    hnp[slot] = __builtin_amdgcn_readfirstlane(hdr[4]);
  }
  auto piece_ml = [&](int piece, int h) { return a.ws_ml + (piece * G + h) * 2; };
  auto piece_o = [&](int piece, int qd) {
    return reinterpret_cast<const f32x4*>(a.ws_o + int64_t(piece) * G * D)[qd];
  };
  // speculative pieces (valid addresses whatever the headers say)
  const int spec[2] = {2 * w + 1, w + 1 < W ? 2 * (w + 1) : 2 * w};
  float sm[2][kQPT], sl[2][kQPT];
  f32x4 so[2][kQPT];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int j = 0; j < kQPT; ++j) {
      const int qd = min(tid + MS::kThreads * j, kQuads - 1);
      const float* ml = piece_ml(spec[c], qd / (D / 4));
      sm[c][j] = ml[0];
      sl[c][j] = ml[1];
      so[c][j] = piece_o(spec[c], qd);
    }
  }
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    if (hvalid[slot] == 0 || (hflags[slot] & kPieceFirst) == 0) continue;
    const int np = min(hnp[slot], W - w);
    const int64_t row0 = int64_t(hseq[slot]) * a.num_q_heads + int64_t(hg[slot]) * G;
#pragma unroll
    for (int j = 0; j < kQPT; ++j) {
      const int qd = tid + MS::kThreads * j;
      if (qd >= kQuads) break;
      const int h = qd / (D / 4);
      // pieces 0 and 1 (from the speculative loads where they match)
      float m0, l0, m1 = -INFINITY, l1 = 0.0f;
      f32x4 o0, o1 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (slot == 1) {
        m0 = sm[0][j];
        l0 = sl[0][j];
        o0 = so[0][j];
      } else {
        m0 = piece_ml(2 * w, h)[0];
        l0 = piece_ml(2 * w, h)[1];
        o0 = piece_o(2 * w, qd);
      }
      if (np > 1) {
        m1 = sm[1][j];
        l1 = sl[1][j];
        o1 = so[1][j];
      }
      float M = fmaxf(m0, m1);
      const float w0 = l0 * __builtin_amdgcn_exp2f(m0 - M);
      const float w1 = np > 1 ? l1 * __builtin_amdgcn_exp2f(m1 - M) : 0.0f;
      float L = w0 + w1;
      f32x4 O = w0 * o0 + w1 * o1;
      // the rest, kBatch at a time, folded in a fixed order; the next
      // batch's loads are issued before the current batch is folded, so a
      // pair of many pieces costs one round trip per batch less
      struct Batch {
        float m[kBatch], l[kBatch];
        f32x4 o[kBatch];
      };
      auto load = [&](Batch& bt, int p0) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int p = p0 + b;
          if (p < np) {
            const float* ml = piece_ml(2 * (w + p), h);
            bt.m[b] = ml[0];
            bt.l[b] = ml[1];
            bt.o[b] = piece_o(2 * (w + p), qd);
          } else {
            bt.m[b] = -INFINITY;
            bt.l[b] = 0.0f;
            bt.o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
      };
      auto fold = [&](const Batch& bt) {
        float Mb = M;
#pragma unroll
        for (int b = 0; b < kBatch; ++b) Mb = fmaxf(Mb, bt.m[b]);
        const float f = __builtin_amdgcn_exp2f(M - Mb);
        L *= f;
        O *= f;
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const float wgt = bt.l[b] * __builtin_amdgcn_exp2f(bt.m[b] - Mb);
          L += wgt;
          O += wgt * bt.o[b];
        }
        M = Mb;
      };
      Batch ba, bb;
      if (np > 2) load(ba, 2);
      for (int p0 = 2; p0 < np; p0 += 2 * kBatch) {
        if (p0 + kBatch < np) load(bb, p0 + kBatch);
        fold(ba);
        if (p0 + kBatch >= np) break;
        if (p0 + 2 * kBatch < np) load(ba, p0 + 2 * kBatch);
        fold(bb);
      }
      store4<DT>(a.out, row0 * D + 4 * qd, O * (1.0f / L));
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed partitions (partition_tokens > 0): one workgroup per (partition, kv
// head, sequence); a sequence longer than one partition leaves one record per
// partition and lse_reduce_kernel merges them.
// ---------------------------------------------------------------------------
template <int DT, int D, int G, bool kTileInBlock>
__global__ __launch_bounds__(kWave * kPartitionWaves) void decode_partition_kernel(DecodeArgs a) {
  constexpr int NW = kPartitionWaves;
  __shared__ SegmentSmem<DT, D, G, NW> sm;
  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int seq = blockIdx.z;
  const int Hq = a.num_q_heads;
  const int T = min(a.context_lens[seq], a.max_context_len);
  const int64_t row0 = int64_t(seq) * Hq + int64_t(g) * G;
  if (T <= 0) {
    if (part == 0) zero_rows<DT, D>(a, row0, G);
    return;
  }
  // partitions of tpp tiles from the tile holding the window's first position
  const int s0 = window_first(T, a.window);
  const int tiles = (T + kTileTokens - 1) / kTileTokens;
  const int tpp = a.partition_tokens / kTileTokens;
  const int lo = s0 / kTileTokens + part * tpp;
  if (lo >= tiles) return;
  const int hi = min(tiles, lo + tpp);
  const int nparts = (attended_tiles(T, a.window) + tpp - 1) / tpp;
  attend_segment<DT, D, G, kTileInBlock, NW>(a, sm, seq, g, T, s0, lo, hi);
  for (int idx = threadIdx.x; idx < G * D; idx += kWave * NW) {
    const int h = idx / D, d = idx - (idx / D) * D;
    float M, L, O;
    merge_waves(sm, h, d, M, L, O);
    if (nparts == 1) {
      store_elem<DT>(a.out, (row0 + h) * D + d, O / L);
    } else {
      const int64_t prow = (row0 + h) * a.num_partitions + part;
      a.ws_o[prow * D + d] = O / L;
      if (d == 0) {
        a.ws_ml[2 * prow] = M;
        a.ws_ml[2 * prow + 1] = L;
      }
    }
  }
}

// log-sum-exp merge of the partitions of one (sequence, kv head) pair:
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
template <int DT, int D, int G>
__global__ __launch_bounds__(kMergeThreads) void lse_reduce_kernel(DecodeArgs a) {
  const int g = blockIdx.x;
  const int seq = blockIdx.y;
  const int T = min(a.context_lens[seq], a.max_context_len);
  const int tpp = a.partition_tokens / kTileTokens;
  const int nparts = (attended_tiles(T, a.window) + tpp - 1) / tpp;
  if (nparts <= 1) return;
  const int NP = a.num_partitions;
  for (int idx = threadIdx.x; idx < G * D; idx += kMergeThreads) {
    const int h = idx / D, d = idx - (idx / D) * D;
    const int64_t row = int64_t(seq) * a.num_q_heads + int64_t(g) * G + h;
    const float* ml = a.ws_ml + 2 * row * NP;
    const float* o = a.ws_o + row * NP * D + d;
    float M = -INFINITY;
#pragma unroll 8
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
    float L = 0.0f, O = 0.0f;
#pragma unroll 8
    for (int p = 0; p < nparts; ++p) {
      const float wgt = ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - M);
      L += wgt;
      O = fmaf(wgt, o[int64_t(p) * D], O);
    }
    store_elem<DT>(a.out, row * D + d, O / L);
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Workgroups of `kernel` the device keeps resident at once (cached per device).
int resident_workgroups(const void* kernel, int kernel_id, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel_id);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) !=
      hipSuccess)
    return 0;
  const int n = std::min(kMaxSplits, std::max(1, cus * std::max(1, per_cu)));
  cache[key] = n;
  return n;
}

template <int DT, int D, int G>
hipError_t launch_decode_g(const DecodeArgs& args, hipStream_t stream) {
  if (args.num_partitions == 0) {
    const DecodeArgs& a = args;
    // balanced split: 16-bit elements, tiles inside one block (checked by the plan)
    if constexpr (DT == PA_F32) {
      return hipErrorInvalidValue;
    } else {
      // variants: appending decode, sliding window, FP8 pools, appending over
      // FP8 pools, plain (one at a time)
      const int mode = a.new_k != nullptr ? (a.kv_fp8 ? 4 : 1) : a.window > 0 ? 2 : a.kv_fp8 ? 3 : 0;
      const void* k =
          mode == 1 ? reinterpret_cast<const void*>(&decode_stream_kernel<DT, D, G, true, false, false>)
          : mode == 2 ? reinterpret_cast<const void*>(&decode_stream_kernel<DT, D, G, false, true, false>)
          : mode == 3 ? reinterpret_cast<const void*>(&decode_stream_kernel<DT, D, G, false, false, true>)
          : mode == 4 ? reinterpret_cast<const void*>(&decode_stream_kernel<DT, D, G, true, false, true>)
                      : reinterpret_cast<const void*>(&decode_stream_kernel<DT, D, G, false, false, false>);
      // The plain, appending and sliding-window variants split the work the
      // same way, so their results agree bit for bit (pa_append_decode equals
      // pa_write_kv + pa_decode): they share one workgroup count, the
      // smallest any of them keeps resident.  The two FP8 variants do the
      // same (pa_append_decode_fp8 equals pa_write_kv_fp8 + pa_decode_fp8).
      const int key = ((DT * 1000 + D) * 100 + G) * 8;
      int W = resident_workgroups(k, key + mode, kWave);
      if (mode >= 3) {
        // FP8 pools, with or without appending: one count for both
        W = std::min(resident_workgroups(reinterpret_cast<const void*>(
                                             &decode_stream_kernel<DT, D, G, false, false, true>),
                                         key + 3, kWave),
                     resident_workgroups(reinterpret_cast<const void*>(
                                             &decode_stream_kernel<DT, D, G, true, false, true>),
                                         key + 4, kWave));
      } else {
        W = std::min({resident_workgroups(reinterpret_cast<const void*>(
                                              &decode_stream_kernel<DT, D, G, false, false, false>),
                                          key + 0, kWave),
                      resident_workgroups(reinterpret_cast<const void*>(
                                              &decode_stream_kernel<DT, D, G, true, false, false>),
                                          key + 1, kWave),
                      resident_workgroups(reinterpret_cast<const void*>(
                                              &decode_stream_kernel<DT, D, G, false, true, false>),
                                          key + 2, kWave)});
      }
      if (W <= 0) return hipErrorInvalidDevice;
      if (mode == 1)
        launch_timed(decode_stream_kernel<DT, D, G, true, false, false>, dim3(W), dim3(kWave),
                         stream, a);
      else if (mode == 2)
        launch_timed(decode_stream_kernel<DT, D, G, false, true, false>, dim3(W), dim3(kWave),
                         stream, a);
      else if (mode == 3)
        launch_timed(decode_stream_kernel<DT, D, G, false, false, true>, dim3(W), dim3(kWave),
                         stream, a);
      else if (mode == 4)
        launch_timed(decode_stream_kernel<DT, D, G, true, false, true>, dim3(W), dim3(kWave),
                         stream, a);
      else
        launch_timed(decode_stream_kernel<DT, D, G, false, false, false>, dim3(W), dim3(kWave),
                         stream, a);
      hipLaunchKernelGGL((merge_pieces_kernel<DT, D, G>), dim3(W),
                         dim3(MergeShape<G, D>::kThreads), 0, stream, a, W);
    }
  } else {
    DecodeArgs a = args;
    if (a.new_k) {
      // fixed partitions read the pools only: write the new rows first
      constexpr int kRowBytes = Geo<DT, D, G>::kRowBytes;
      const int64_t chunks = int64_t(2) * a.num_seqs * a.num_kv_heads * (kRowBytes / 16);
      const int blocks = int(std::min<int64_t>((chunks + 255) / 256, 4096));
      hipLaunchKernelGGL(append_kv_kernel, dim3(blocks), dim3(256), 0, stream, a, kRowBytes);
      a.new_k = nullptr;
      a.new_v = nullptr;
    }
    const dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
    // a 16-token tile lies inside one block when the block size is a multiple of 16
    if (a.log2_block >= 4) {
      launch_timed(decode_partition_kernel<DT, D, G, true>, grid,
                       dim3(kWave * kPartitionWaves), stream, a);
    } else {
      launch_timed(decode_partition_kernel<DT, D, G, false>, grid,
                       dim3(kWave * kPartitionWaves), stream, a);
    }
    if (a.num_partitions > 1) {
      const dim3 rgrid(a.num_kv_heads, a.num_seqs);
      hipLaunchKernelGGL((lse_reduce_kernel<DT, D, G>), rgrid, dim3(kMergeThreads), 0,
                         stream, a);
    }
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_decode_d(const DecodeArgs& a, int32_t group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_decode_g<DT, D, 1>(a, stream);
    case 2: return launch_decode_g<DT, D, 2>(a, stream);
    case 3: return launch_decode_g<DT, D, 3>(a, stream);
    case 4: return launch_decode_g<DT, D, 4>(a, stream);
    case 5: return launch_decode_g<DT, D, 5>(a, stream);
    case 6: return launch_decode_g<DT, D, 6>(a, stream);
    case 7: return launch_decode_g<DT, D, 7>(a, stream);
    case 8: return launch_decode_g<DT, D, 8>(a, stream);
    case 16: return launch_decode_g<DT, D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_decode_dt(const DecodeArgs& a, int32_t head_dim, int32_t group,
                            hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_decode_d<DT, 64>(a, group, stream);
    case 128: return launch_decode_d<DT, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Library-held decode workspace for callers that cannot allocate
// (pa_decode_noalloc).  One copy per GPU, living until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device may reach a
// kernel or a copy.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;          // device -> that device's copy
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  addr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

KernelTimer& kernel_timer() {
  static KernelTimer t;
  return t;
}

void profile_start() {
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> lock(t.mu);
  t.on.store(true);
}

hipError_t profile_stop(int32_t* launches, double* mean_us) {
  KernelTimer& t = kernel_timer();
  std::lock_guard<std::mutex> lock(t.mu);
  t.on.store(false);
  hipError_t err = hipSuccess;
  double total_ms = 0.0;
  int32_t n = 0;
  for (auto& e : t.events) {
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventSynchronize(e.second);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e.first, e.second);
    if (err == hipSuccess) {
      total_ms += ms;
      ++n;
    }
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  t.events.clear();
  *launches = n;
  *mean_us = n ? total_ms * 1e3 / n : 0.0;
  return err;
}


hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(write_kv_kernel, dim3(a.num_tokens), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_write_kv_fp8(const WriteArgs& a, int32_t dtype, float k_scale, float v_scale,
                               hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  switch (dtype) {
    case PA_F32:
      hipLaunchKernelGGL(write_kv_fp8_kernel<PA_F32>, dim3(a.num_tokens), dim3(256), 0, stream, a,
                         k_scale, v_scale);
      break;
    case PA_F16:
      hipLaunchKernelGGL(write_kv_fp8_kernel<PA_F16>, dim3(a.num_tokens), dim3(256), 0, stream, a,
                         k_scale, v_scale);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(write_kv_fp8_kernel<PA_BF16>, dim3(a.num_tokens), dim3(256), 0, stream,
                         a, k_scale, v_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int32_t dtype, int32_t head_dim, int32_t group,
                         hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (dtype) {
    case PA_F32: return launch_decode_dt<PA_F32>(a, head_dim, group, stream);
    case PA_F16: return launch_decode_dt<PA_F16>(a, head_dim, group, stream);
    case PA_BF16: return launch_decode_dt<PA_BF16>(a, head_dim, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa

// HIP kernels for gfx950 (CDNA4): the paged KV slot write and paged decode
// attention with a log-sum-exp merge of context partitions.
//
// Address rule ("vLLM Framework and Inference Engine Design", section "What is
// the essence of vLLM's PagedAttention?"): token t of a sequence is in physical
// block table[t >> log2B] at offset t & (B-1).  Pools are
// [num_blocks][num_kv_heads][B][D]: one (block, kv head) pair is B*D
// contiguous elements, so every row of D elements is read with 16-byte loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kWave = 64;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kWave * kDecodeWaves;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
template <int DT> struct Elem;
template <> struct Elem<PA_F32> { static constexpr int kPerChunk = 4; };
template <> struct Elem<PA_F16> { static constexpr int kPerChunk = 8; };
template <> struct Elem<PA_BF16> { static constexpr int kPerChunk = 8; };

// 16-byte chunk -> float32 values
template <int DT> __device__ inline void unpack(const uint4& c, float* f);

template <> __device__ inline void unpack<PA_F32>(const uint4& c, float* f) {
  f[0] = __uint_as_float(c.x);
  f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z);
  f[3] = __uint_as_float(c.w);
}

template <> __device__ inline void unpack<PA_F16>(const uint4& c, float* f) {
  const f16x8 h = __builtin_bit_cast(f16x8, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(h[e]);
}

// a bfloat16 is the high half of a float32
template <> __device__ inline void unpack<PA_BF16>(const uint4& c, float* f) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// float32 -> element, round to nearest even
template <int DT> __device__ inline void store_elem(void* base, size_t idx, float x);

template <> __device__ inline void store_elem<PA_F32>(void* base, size_t idx, float x) {
  static_cast<float*>(base)[idx] = x;
}

template <> __device__ inline void store_elem<PA_F16>(void* base, size_t idx, float x) {
  static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
}

template <> __device__ inline void store_elem<PA_BF16>(void* base, size_t idx, float x) {
  uint32_t u = __float_as_uint(x);
  uint16_t r;
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    r = static_cast<uint16_t>((u >> 16) | 0x0040u);            // quiet NaN
  } else {
    r = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  static_cast<uint16_t*>(base)[idx] = r;
}

// ---------------------------------------------------------------------------
// QK^T tile on the matrix cores: 16 query rows x 16 keys, k = one 16-byte
// chunk per lane group.  A and B take their k index from the same
// (lane group, element) position, so the contraction pairs q[d] with k[d]
// whatever order the hardware gives k inside one instruction.
// ---------------------------------------------------------------------------
template <int DT> __device__ inline f32x4 mfma_chunk(const uint4& a, const uint4& b, f32x4 acc);

template <> __device__ inline f32x4 mfma_chunk<PA_BF16>(const uint4& a, const uint4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <> __device__ inline f32x4 mfma_chunk<PA_F16>(const uint4& a, const uint4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

template <> __device__ inline f32x4 mfma_chunk<PA_F32>(const uint4& a, const uint4& b, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------------------
// reductions across the 16 lanes of a DPP row (all lanes get the result)
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within the row

template <int CTRL> __device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

__device__ inline float row_sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
template <int DT, int D, int G>
struct Geo {
  static constexpr int EPC = Elem<DT>::kPerChunk;   // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;               // chunks per row
  static constexpr int KK = CPR / 4;                // key chunks per lane per tile
  static constexpr int RPI = kWave / CPR;           // value rows per load instruction
  static constexpr int VS = kTileTokens / RPI;      // value loads per lane per tile
  static constexpr int NHB = (G + 3) / 4;           // batches of four query heads
  static constexpr int kRowBytes = D * (16 / EPC);
  static_assert(CPR % 4 == 0 && kWave % CPR == 0 && kTileTokens % RPI == 0, "shape");
};

template <int DT, int D, int G>
struct SegmentSmem {
  f32x4 p[kDecodeWaves][kTileTokens][Geo<DT, D, G>::NHB];
  float m[kDecodeWaves][G];
  float l[kDecodeWaves][G];
  float o[kDecodeWaves][G][D];
};

// Attend over tiles [tile_lo, tile_hi) (at least one) of pair (seq, g) whose
// sequence holds T > 0 tokens.  Ends with a workgroup barrier after which
// sm.m / sm.l / sm.o hold every wave's max, sum and unnormalised output.
template <int DT, int D, int G, bool kTileInBlock>
__device__ void attend_segment(const DecodeArgs& a, SegmentSmem<DT, D, G>& sm, int seq, int g,
                               int T, int tile_lo, int tile_hi) {
  using GE = Geo<DT, D, G>;
  constexpr int EPC = GE::EPC, CPR = GE::CPR, KK = GE::KK, RPI = GE::RPI, VS = GE::VS;
  constexpr int NHB = GE::NHB, kRowBytes = GE::kRowBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gq = lane >> 4;
  const int c = lane & 15;
  const int rho = lane / CPR;
  const int chi = lane % CPR;
  const int Hq = a.num_q_heads;
  const int hq0 = g * G;

  // query A operands: row c carries head 4*hb + (c & 3); heads >= G are zero
  uint4 qa[NHB][KK];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int head = 4 * hb + (c & 3);
    const int head_ld = head < G ? head : G - 1;   // padding rows never dereference
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + (int64_t(seq) * Hq + hq0 + head_ld) * kRowBytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qa[hb][kk] = head < G ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
  }

  const int lb = a.log2_block;
  const int bmask = (1 << lb) - 1;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq;
  const int64_t head_rows = int64_t(g) << lb;                 // kv head g inside a block
  const int64_t blk_rows = int64_t(a.num_kv_heads) << lb;     // rows per block
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int nblk = a.num_blocks;

  const int span = tile_hi - tile_lo - wave;
  const int nmine = span > 0 ? (span + kDecodeWaves - 1) / kDecodeWaves : 0;

  // block ids of this wave's tiles, 64 tiles per load: lane j holds the block
  // of the wave's tile 64*batch + j (used when a tile lies inside one block)
  int tbl = 0;
  auto load_tbl = [&](int batch) {
    const int k = min(64 * batch + lane, nmine - 1);
    const int t = min((tile_lo + wave + kDecodeWaves * k) * kTileTokens, T - 1);
    tbl = min(max(table[t >> lb], 0), nblk - 1);
  };

  struct Regs {
    uint4 k[KK];
    uint4 v[VS];
  };
  // Tokens past T-1 (the tail of the sequence's last tile) read row T-1: finite
  // data, never a slot outside the sequence; their probability is zero.
  auto load_tile = [&](int kidx, Regs& r) {
    const int t0 = (tile_lo + wave + kDecodeWaves * kidx) * kTileTokens;
    const int last = T - 1 - t0;
    if constexpr (kTileInBlock) {
      const int64_t blk = __builtin_amdgcn_readlane(tbl, kidx & 63);
      const int64_t row0 = blk * blk_rows + head_rows + (t0 & bmask);
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + (row0 + min(c, last)) * kRowBytes);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) r.k[kk] = kp[4 * kk + gq];
#pragma unroll
      for (int s = 0; s < VS; ++s)
        r.v[s] = reinterpret_cast<const uint4*>(
            vbase + (row0 + min(s * RPI + rho, last)) * kRowBytes)[chi];
    } else {
      auto row_of = [&](int dt) -> int64_t {
        const int t = t0 + min(dt, last);
        const int64_t blk = min(max(table[t >> lb], 0), nblk - 1);
        return blk * blk_rows + head_rows + (t & bmask);
      };
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + row_of(c) * kRowBytes);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) r.k[kk] = kp[4 * kk + gq];
#pragma unroll
      for (int s = 0; s < VS; ++s)
        r.v[s] = reinterpret_cast<const uint4*>(vbase + row_of(s * RPI + rho) * kRowBytes)[chi];
    }
  };

  float m_run[NHB][4], l_run[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[hb][i] = -INFINITY;
      l_run[hb][i] = 0.0f;
    }
  float acc[G][EPC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;

  auto compute_tile = [&](int kidx, const Regs& r) {
    const int t0 = (tile_lo + wave + kDecodeWaves * kidx) * kTileTokens;
    const bool valid = t0 + c < T;
    float pr[NHB][4], alpha[NHB][4];
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
        pr[hb][i] = __builtin_amdgcn_exp2f(s - m_use);
        l_run[hb][i] = l_run[hb][i] * alpha[hb][i] + pr[hb][i];
        m_run[hb][i] = m_new;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h / 4][h % 4];

    if (gq == 0) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        sm.p[wave][c][hb] = f32x4{pr[hb][0], pr[hb][1], pr[hb][2], pr[hb][3]};
    }
    wave_sync_lds();
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      float v[EPC];
      unpack<DT>(r.v[s], v);
      const int row = s * RPI + rho;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4 pp = sm.p[wave][row][hb];
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
  };

  if (nmine > 0) {
    if constexpr (kTileInBlock) load_tbl(0);
    Regs A, B;
    load_tile(0, A);
    for (int k = 0; k < nmine; k += 2) {
      if (k + 1 < nmine) {
        if (kTileInBlock && ((k + 1) & 63) == 0) load_tbl((k + 1) >> 6);
        load_tile(k + 1, B);
      }
      compute_tile(k, A);
      if (k + 1 >= nmine) break;
      if (k + 2 < nmine) {
        if (kTileInBlock && ((k + 2) & 63) == 0) load_tbl((k + 2) >> 6);
        load_tile(k + 2, A);
      }
      compute_tile(k + 1, B);
    }
  }

  // wave totals: l summed over the 16 token lanes, acc over the value rows
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
  if (lane == 0) {
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
  __syncthreads();
}

// Merge the four waves' results for (head h, element d): M = max, L = sum of
// 2^(m_w - M) l_w, O = sum of 2^(m_w - M) o_w.  The attention output is O / L.
template <int DT, int D, int G>
__device__ inline void merge_waves(const SegmentSmem<DT, D, G>& sm, int h, int d, float& M,
                                   float& L, float& O) {
  M = sm.m[0][h];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm.m[w][h]);
  L = 0.0f;
  O = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) {
    const float f = __builtin_amdgcn_exp2f(sm.m[w][h] - M);
    L = fmaf(f, sm.l[w][h], L);
    O = fmaf(f, sm.o[w][h][d], O);
  }
}

template <int DT, int D>
__device__ inline void zero_rows(const DecodeArgs& a, int64_t row0, int nrows) {
  for (int i = threadIdx.x; i < nrows * D; i += kDecodeThreads)
    store_elem<DT>(a.out, row0 * D + i, 0.0f);
}

// ---------------------------------------------------------------------------
// Balanced split (the default).  The grid holds as many workgroups as the GPU
// keeps resident.  The flattened work (sequence, kv head, tile) is cut into
// equal contiguous shares, one per workgroup, so long and short sequences
// load every workgroup alike.  A pair cut by a share boundary leaves one
// "piece" per workgroup it touches: (max, sum, normalised output) per head in
// slot 0 (the share's first segment) or slot 1 (its last), and the piece
// merge kernel combines them.  Pairs inside one share are written directly.
// ---------------------------------------------------------------------------
constexpr int kPieceFirst = 1;   // the piece starts at the pair's first tile
constexpr int kPieceLast = 2;    // the piece ends at the pair's last tile

template <int DT, int D, int G, bool kTileInBlock>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(DecodeArgs a) {
  __shared__ SegmentSmem<DT, D, G> sm;
  __shared__ int32_t s_len[kMaxSplitSeqs];
  __shared__ long long s_wsum[kDecodeWaves];
  __shared__ long long s_start[2];

  const int w = blockIdx.x;
  const int W = gridDim.x;
  const int N = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  if (tid < 2) a.ws_hdr[(2 * w + tid) * 4] = 0;   // both piece slots empty so far

  // clamped lengths into LDS; tiles of this thread's run of sequences
  const int chunk = (N + kDecodeThreads - 1) / kDecodeThreads;
  const int i0 = min(N, tid * chunk);
  const int i1 = min(N, i0 + chunk);
  long long mine = 0;
  for (int i = i0; i < i1; ++i) {
    const int T = min(max(a.context_lens[i], 0), a.max_context_len);
    s_len[i] = T;
    mine += (T + kTileTokens - 1) / kTileTokens;
  }
  long long incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  long long before = 0, all_tiles = 0;
#pragma unroll
  for (int i = 0; i < kDecodeWaves; ++i) {
    before += i < wave ? s_wsum[i] : 0;
    all_tiles += s_wsum[i];
  }
  const long long excl = before + incl - mine;

  // zero-length sequences get zero rows (spread over every workgroup)
  for (int s = w; s < N; s += W)
    if (s_len[s] == 0) zero_rows<DT, D>(a, int64_t(s) * Hq, Hq);

  const long long total = all_tiles * Hkv;
  const long long want = (total + a.min_split_tiles - 1) / a.min_split_tiles;
  const int Weff = int(max(1LL, min(static_cast<long long>(W), want)));
  if (w >= Weff) return;
  const long long lo = total * w / Weff;
  const long long hi = total * (w + 1) / Weff;
  if (lo >= hi) return;
  if (mine > 0 && lo >= excl * Hkv && lo < (excl + mine) * Hkv) {
    long long cum = excl;
    for (int i = i0; i < i1; ++i) {
      const int t = (s_len[i] + kTileTokens - 1) / kTileTokens;
      if (lo < (cum + t) * Hkv) {
        s_start[0] = i;
        s_start[1] = cum;
        break;
      }
      cum += t;
    }
  }
  __syncthreads();

  int s = int(s_start[0]);
  long long cum = s_start[1];
  long long pos = lo;
  while (pos < hi && s < N) {
    const int T = s_len[s];
    const int tiles = (T + kTileTokens - 1) / kTileTokens;
    const long long base = cum * Hkv;
    if (pos >= base + static_cast<long long>(tiles) * Hkv) {
      cum += tiles;
      ++s;
      continue;
    }
    const long long r = pos - base;
    const int g = int(r / tiles);
    const int tile0 = int(r - static_cast<long long>(g) * tiles);
    const long long seg_end = min(hi, base + static_cast<long long>(g + 1) * tiles);
    const int tile1 = tile0 + int(seg_end - pos);
    attend_segment<DT, D, G, kTileInBlock>(a, sm, s, g, T, tile0, tile1);

    const int flags = (tile0 == 0 ? kPieceFirst : 0) | (tile1 == tiles ? kPieceLast : 0);
    const int64_t row0 = int64_t(s) * Hq + int64_t(g) * G;
    if (flags == (kPieceFirst | kPieceLast)) {
      for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
        const int h = idx / D, d = idx - (idx / D) * D;
        float M, L, O;
        merge_waves(sm, h, d, M, L, O);
        store_elem<DT>(a.out, (row0 + h) * D + d, O / L);
      }
    } else {
      const int piece = 2 * w + (pos == lo ? 0 : 1);
      for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
        const int h = idx / D, d = idx - (idx / D) * D;
        float M, L, O;
        merge_waves(sm, h, d, M, L, O);
        a.ws_o[(int64_t(piece) * G + h) * D + d] = O / L;
        if (d == 0) {
          a.ws_ml[(piece * G + h) * 2] = M;
          a.ws_ml[(piece * G + h) * 2 + 1] = L;
        }
      }
      if (tid == 0) {
        int32_t* hdr = a.ws_hdr + piece * 4;
        hdr[1] = s;
        hdr[2] = g;
        hdr[3] = flags;
        hdr[0] = 1;
      }
    }
    __syncthreads();       // sm is reused by the next segment
    pos = seg_end;
  }
}

// Combine the pieces of every pair that starts inside this workgroup's share
// and continues into the next shares (slot 0 of the following workgroups,
// up to the piece that holds the pair's last tile).
template <int DT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void merge_pieces_kernel(DecodeArgs a) {
  const int w = blockIdx.x;
  const int W = gridDim.x;
  for (int slot = 0; slot < 2; ++slot) {
    const int32_t* hdr = a.ws_hdr + (2 * w + slot) * 4;
    if (hdr[0] == 0 || (hdr[3] & kPieceFirst) == 0) continue;
    const int seq = hdr[1];
    const int g = hdr[2];
    const int64_t row0 = int64_t(seq) * a.num_q_heads + int64_t(g) * G;
    for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
      const int h = idx / D, d = idx - (idx / D) * D;
      float M = -INFINITY, L = 0.0f, O = 0.0f;
      int piece = 2 * w + slot;
      for (int ww = w; ww < W; ++ww) {
        const float m = a.ws_ml[(piece * G + h) * 2];
        const float l = a.ws_ml[(piece * G + h) * 2 + 1];
        const float o = a.ws_o[(int64_t(piece) * G + h) * D + d];
        const int fl = a.ws_hdr[piece * 4 + 3];
        const float M2 = fmaxf(M, m);
        const float f_old = __builtin_amdgcn_exp2f(M - M2);
        const float f_new = l * __builtin_amdgcn_exp2f(m - M2);
        L = L * f_old + f_new;
        O = O * f_old + f_new * o;
        M = M2;
        if (fl & kPieceLast) break;
        piece = 2 * (ww + 1);
      }
      store_elem<DT>(a.out, (row0 + h) * D + d, O / L);
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed partitions (partition_tokens > 0): one workgroup per (partition, kv
// head, sequence); a sequence longer than one partition leaves one record per
// partition and lse_reduce_kernel merges them.
// ---------------------------------------------------------------------------
template <int DT, int D, int G, bool kTileInBlock>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeArgs a) {
  __shared__ SegmentSmem<DT, D, G> sm;
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
  const int tiles = (T + kTileTokens - 1) / kTileTokens;
  const int tpp = a.partition_tokens / kTileTokens;
  const int lo = part * tpp;
  if (lo >= tiles) return;
  const int hi = min(tiles, lo + tpp);
  const int nparts = (tiles + tpp - 1) / tpp;
  attend_segment<DT, D, G, kTileInBlock>(a, sm, seq, g, T, lo, hi);
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
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
__global__ __launch_bounds__(kDecodeThreads) void lse_reduce_kernel(DecodeArgs a) {
  const int g = blockIdx.x;
  const int seq = blockIdx.y;
  const int T = min(a.context_lens[seq], a.max_context_len);
  const int P = a.partition_tokens;
  const int nparts = T > 0 ? (T + P - 1) / P : 0;
  if (nparts <= 1) return;
  const int NP = a.num_partitions;
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
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
// Workgroups of `kernel` the device keeps resident at once (cached per device).
int resident_workgroups(const void* kernel, int kernel_id) {
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeThreads, 0) !=
      hipSuccess)
    return 0;
  const int n = std::min(kMaxSplits, std::max(1, cus * std::max(1, per_cu)));
  cache[key] = n;
  return n;
}

template <int DT, int D, int G, bool kTileInBlock>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_partitions == 0) {          // balanced split
    const void* k = reinterpret_cast<const void*>(&decode_split_kernel<DT, D, G, kTileInBlock>);
    const int W = resident_workgroups(k, (DT * 1000 + D) * 100 + G * 2 + (kTileInBlock ? 1 : 0));
    if (W <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL((decode_split_kernel<DT, D, G, kTileInBlock>), dim3(W),
                       dim3(kDecodeThreads), 0, stream, a);
    hipLaunchKernelGGL((merge_pieces_kernel<DT, D, G>), dim3(W), dim3(kDecodeThreads), 0,
                       stream, a);
  } else {
    const dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, kTileInBlock>), grid,
                       dim3(kDecodeThreads), 0, stream, a);
    if (a.num_partitions > 1) {
      const dim3 rgrid(a.num_kv_heads, a.num_seqs);
      hipLaunchKernelGGL((lse_reduce_kernel<DT, D, G>), rgrid, dim3(kDecodeThreads), 0,
                         stream, a);
    }
  }
  return hipGetLastError();
}

template <int DT, int D, int G>
hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
  // a 16-token tile lies inside one block when the block size is a multiple of 16
  if (a.log2_block >= 4) return launch_decode_t<DT, D, G, true>(a, stream);
  return launch_decode_t<DT, D, G, false>(a, stream);
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

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(write_kv_kernel, dim3(a.num_tokens), dim3(256), 0, stream, a);
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

// HIP kernels for gfx950 (CDNA4): the paged KV slot write and paged decode
// attention with a log-sum-exp merge of context partitions.
//
// Address rule ("vLLM Framework and Inference Engine Design", section "What is
// the essence of vLLM's PagedAttention?"): token t of a sequence is in physical
// block table[t >> log2B] at offset t & (B-1).  Pools are
// [num_blocks][num_kv_heads][B][D]: one (block, kv head) pair is B*D
// contiguous elements, so every row of D elements is read with 16-byte loads.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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
// decode: one workgroup per (context partition, kv head, sequence)
//
// Each of the 4 waves takes every 4th 16-token tile of the partition.
//   K side: lane (gq = lane/16, c = lane%16) loads 16-byte chunks
//     gq, gq+4, ... of token c's key row: the B operand of a 16x16 MFMA whose
//     A operand holds the G query heads of this kv head, repeated down the 16
//     rows.  Lane (gq, c) then holds token c's scores for four heads.
//   V side: lane (rho = lane/CPR, chi = lane%CPR) loads chunk chi of value
//     rows rho, rho+RPI, ...; it accumulates G x (elements per chunk) sums.
//   The probabilities go through a 16 x G float LDS tile per wave.
// Online softmax in the exp2 domain: m = running max, l = running sum.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeArgs a) {
  constexpr int EPC = Elem<DT>::kPerChunk;     // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                 // chunks per row
  constexpr int KK = CPR / 4;                  // key chunks per lane per tile
  constexpr int RPI = kWave / CPR;             // value rows per load instruction
  constexpr int VS = kTileTokens / RPI;        // value loads per lane per tile
  constexpr int NHB = (G + 3) / 4;             // batches of four query heads
  static_assert(CPR % 4 == 0 && kWave % CPR == 0 && kTileTokens % RPI == 0, "shape");

  __shared__ int32_t s_table[kTableSliceCap];
  __shared__ f32x4 s_p[kDecodeWaves][kTileTokens][NHB];
  __shared__ float s_m[kDecodeWaves][G];
  __shared__ float s_l[kDecodeWaves][G];
  __shared__ float s_o[kDecodeWaves][G][D];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int hq0 = g * G;
  const int Hq = a.num_q_heads;

  // lengths outside [0, max_context_len] are clamped so no access leaves the
  // grid's partitions or the workspace
  const int T = min(a.context_lens[seq], a.max_context_len);
  if (T <= 0) {
    if (part == 0) {
      for (int i = tid; i < G * D; i += kDecodeThreads)
        store_elem<DT>(a.out, (int64_t(seq) * Hq + hq0) * D + i, 0.0f);
    }
    return;
  }
  const int P = a.partition_tokens;
  const int tok0 = part * P;
  if (tok0 >= T) return;
  const int tok1 = min(T, tok0 + P);
  const int nparts = (T + P - 1) / P;
  const int lb = a.log2_block;
  const int bmask = (1 << lb) - 1;
  const int j0 = tok0 >> lb;
  const int nj = ((tok1 - 1) >> lb) - j0 + 1;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq;
  for (int i = tid; i < nj; i += kDecodeThreads) s_table[i] = table[j0 + i];

  const int gq = lane >> 4;
  const int c = lane & 15;
  const int rho = lane / CPR;
  const int chi = lane % CPR;

  // query A operands: row c carries head 4*hb + (c & 3); heads >= G are zero
  uint4 qa[NHB][KK];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int head = 4 * hb + (c & 3);
    const int head_ld = head < G ? head : G - 1;   // padding rows never dereference
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + ((int64_t(seq) * Hq + hq0 + head_ld) * D) * (16 / EPC));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qa[hb][kk] = head < G ? qrow[4 * kk + gq] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int64_t kv_stride_blk = int64_t(a.num_kv_heads) << lb;   // rows per block
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  constexpr int kRowBytes = D * (16 / EPC);

  // byte offset of the row of token t (clamped into this partition)
  auto row_off = [&](int t) -> int64_t {
    const int tc = min(t, tok1 - 1);
    const int64_t blk = min(max(s_table[(tc >> lb) - j0], 0), a.num_blocks - 1);
    return ((blk * kv_stride_blk) + (int64_t(g) << lb) + (tc & bmask)) * kRowBytes;
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

  const int ntiles = (tok1 - tok0 + kTileTokens - 1) / kTileTokens;
  for (int it = wave; it < ntiles; it += kDecodeWaves) {
    const int tbase = tok0 + it * kTileTokens;
    uint4 kreg[KK];
    {
      const uint4* krow = reinterpret_cast<const uint4*>(kbase + row_off(tbase + c));
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kreg[kk] = krow[4 * kk + gq];
    }
    uint4 vreg[VS];
#pragma unroll
    for (int s = 0; s < VS; ++s)
      vreg[s] = reinterpret_cast<const uint4*>(vbase + row_off(tbase + s * RPI + rho))[chi];

    const bool valid = (tbase + c) < tok1;
    float pr[NHB][4], alpha[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = mfma_chunk<DT>(qa[hb][kk], kreg[kk], sc);
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
        s_p[wave][c][hb] = f32x4{pr[hb][0], pr[hb][1], pr[hb][2], pr[hb][3]};
    }
    wave_sync_lds();
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      float v[EPC];
      unpack<DT>(vreg[s], v);
      const int row = s * RPI + rho;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4 pp = s_p[wave][row][hb];
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

  // per-wave totals: sum l over the 16 token lanes, sum acc over value rows
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
      s_m[wave][h] = m_run[h / 4][h % 4];
      s_l[wave][h] = l_run[h / 4][h % 4];
    }
  }
  if (rho == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) s_o[wave][h][chi * EPC + e] = acc[h][e];
  }
  __syncthreads();

  // merge the four waves, then either finish or park the partial result
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
      L = fmaf(f, s_l[w][h], L);
      O = fmaf(f, s_o[w][h][d], O);
    }
    const int64_t row = int64_t(seq) * Hq + hq0 + h;
    if (nparts == 1) {
      store_elem<DT>(a.out, row * D + d, O / L);
    } else {
      const int64_t prow = row * a.num_partitions + part;
      a.ws_o[prow * D + d] = O / L;
      if (d == 0) {
        a.ws_ml[2 * prow] = M;
        a.ws_ml[2 * prow + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of the context partitions of one (sequence, query head)
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(D) void lse_reduce_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const int T = min(a.context_lens[seq], a.max_context_len);
  const int P = a.partition_tokens;
  const int nparts = T > 0 ? (T + P - 1) / P : 0;
  if (nparts <= 1) return;
  const int64_t row = int64_t(seq) * a.num_q_heads + hq;
  const float* ml = a.ws_ml + 2 * row * a.num_partitions;
  const float* o = a.ws_o + row * a.num_partitions * D;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.0f, O = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float w = ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - M);
    L += w;
    O = fmaf(w, o[p * D + d], O);
  }
  store_elem<DT>(a.out, row * D + d, O / L);
}

template <int DT, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, G>), grid, dim3(kDecodeThreads), 0, stream, a);
  if (a.num_partitions > 1) {
    const dim3 rgrid(a.num_q_heads, a.num_seqs);
    hipLaunchKernelGGL((lse_reduce_kernel<DT, D>), rgrid, dim3(D), 0, stream, a);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_decode_d(const DecodeArgs& a, int32_t group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_decode_t<DT, D, 1>(a, stream);
    case 2: return launch_decode_t<DT, D, 2>(a, stream);
    case 3: return launch_decode_t<DT, D, 3>(a, stream);
    case 4: return launch_decode_t<DT, D, 4>(a, stream);
    case 5: return launch_decode_t<DT, D, 5>(a, stream);
    case 6: return launch_decode_t<DT, D, 6>(a, stream);
    case 7: return launch_decode_t<DT, D, 7>(a, stream);
    case 8: return launch_decode_t<DT, D, 8>(a, stream);
    case 16: return launch_decode_t<DT, D, 16>(a, stream);
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

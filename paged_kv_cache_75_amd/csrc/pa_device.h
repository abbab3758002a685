// Device helpers shared by the attention sources (decode and write kernels in
// pa_kernels.hip, chunked prefill in pa_prefill.hip): the wave size, buffer
// descriptors, element types and their 16-byte chunks, matrix-core wrappers,
// the tile geometry of a [blocks][kv heads][B][D] pool, and LDS types for
// transposed reads.  Internal linkage: every source gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kWave = 64;
// raw buffer descriptor, word 3 for gfx9-family chips: 32-bit data format,
// no swizzle; loads past num_records return zero
constexpr int kBufferDword3 = 0x00020000;

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

// four consecutive outputs (one 8- or 16-byte store)
template <int DT> __device__ inline void store4(void* base, int64_t idx, f32x4 x);
template <> __device__ inline void store4<PA_F32>(void* base, int64_t idx, f32x4 x) {
  *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = x;
}
template <> __device__ inline void store4<PA_F16>(void* base, int64_t idx, f32x4 x) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 h = {static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]),
                static_cast<_Float16>(x[2]), static_cast<_Float16>(x[3])};
  *reinterpret_cast<h4*>(static_cast<_Float16*>(base) + idx) = h;
}
template <> __device__ inline void store4<PA_BF16>(void* base, int64_t idx, f32x4 x) {
  // round to nearest even (gfx950 converts a pair per instruction; NaN stays NaN)
  typedef __bf16 b4 __attribute__((ext_vector_type(4)));
  const b4 h = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]), static_cast<__bf16>(x[2]),
                static_cast<__bf16>(x[3])};
  *reinterpret_cast<b4*>(static_cast<__bf16*>(base) + idx) = h;
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

// Inclusive prefix sum over the 64 lanes of a wave on the vector ALU (DPP):
// shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row add 0), then row 0's total into row 1 and row 2's total into
// row 3 (lane 15's and lane 47's values, broadcast), then lane 31's total into
// rows 2 and 3.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}
// the value of the last lane (the total after wave_scan_incl)
__device__ __forceinline__ int wave_last(int x) { return __builtin_amdgcn_readlane(x, kWave - 1); }

// The maximum (sum) over the four lanes c, c + 16, c + 32, c + 48 of a column:
// row swaps on the vector ALU rather than permutes through LDS.  The sum adds
// the pairs (rows 0 + 1) and (rows 2 + 3) first, in the same order on every
// lane.
__device__ __forceinline__ float column_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float column_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

template <int DT, int D>
struct KeyRegs {
  uint4 k[Geo<DT, D, 1>::KK];
};
template <int DT, int D>
struct ValRegs {
  uint4 v[Geo<DT, D, 1>::VS];
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef _Float16 v4f16 __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

template <int DT> __device__ inline f32x4 mfma_pv(v4i16 a, v4i16 b, f32x4 acc);
template <> __device__ inline f32x4 mfma_pv<PA_BF16>(v4i16 a, v4i16 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
template <> __device__ inline f32x4 mfma_pv<PA_F16>(v4i16 a, v4i16 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4f16, a),
                                               __builtin_bit_cast(v4f16, b), acc, 0, 0, 0);
}

template <int DT> __device__ inline v4i16 pack4(const float* p);
template <> __device__ inline v4i16 pack4<PA_BF16>(const float* p) {
  const v4bf16 x = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                    static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
  return __builtin_bit_cast(v4i16, x);
}
template <> __device__ inline v4i16 pack4<PA_F16>(const float* p) {
  const v4f16 x = {static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]),
                   static_cast<_Float16>(p[2]), static_cast<_Float16>(p[3])};
  return __builtin_bit_cast(v4i16, x);
}

}  // namespace

}  // namespace pa

// Device-side building blocks shared by the library's gfx950 kernels:
// element types, 16-byte row loads, widening to fp32, wavefront reductions
// and block translation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------- element types
// Storage tags. Every cache row is moved as 16-byte vectors; a lane widens
// its vector to fp32 in registers.
struct F32 {
  static constexpr int kBytes = 4;
};
struct F16 {
  static constexpr int kBytes = 2;
};
struct BF16 {
  static constexpr int kBytes = 2;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret one 32-bit word as two packed 16-bit values. The word is taken
// by value on purpose: __builtin_bit_cast applied directly to an element of
// an ext_vector_type (v[j], v.y) reads element 0 with this compiler.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

template <typename T>
struct Vec {
  static constexpr int kElems = 16 / T::kBytes;  // elements per 16-byte vector
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load: the row is read once, so it is marked non-temporal and
// does not displace reusable lines in the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Widen the 16-byte vector to fp32: element j of the vector -> out[j].
__device__ __forceinline__ void widen(F32, u32x4 v, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(v[j]);
}

__device__ __forceinline__ void widen(BF16, u32x4 v, float* out) {
  // bfloat16 is the upper half of an fp32 pattern: widening is a shift.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(v[j] << 16);
    out[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void widen(F16, u32x4 v, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 h = as_f16x2(v[j]);
    out[2 * j] = static_cast<float>(h[0]);
    out[2 * j + 1] = static_cast<float>(h[1]);
  }
}

// Partial dot product of two 16-byte vectors, accumulated in fp32.
__device__ __forceinline__ float dot16(F32, u32x4 a, u32x4 b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(__uint_as_float(a[j]), __uint_as_float(b[j]), acc);
  return acc;
}

__device__ __forceinline__ float dot16(BF16, u32x4 a, u32x4 b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[j]), as_bf16x2(b[j]), acc, false);
  return acc;
}

__device__ __forceinline__ float dot16(F16, u32x4 a, u32x4 b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2(as_f16x2(a[j]), as_f16x2(b[j]), acc, false);
  return acc;
}

// Narrow fp32 to the storage type, round to nearest even.
__device__ __forceinline__ uint32_t narrow_bits(BF16, float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // keep NaN quiet
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t narrow_bits(F16, float x) {
  _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------- reductions
// DPP lane patterns inside one 16-lane row of a wavefront.
enum : int {
  kDppQuadSwap1 = 0xB1,    // quad_perm [1,0,3,2]: partner lane ^ 1
  kDppQuadSwap2 = 0x4E,    // quad_perm [2,3,0,1]: partner lane ^ 2
  kDppHalfMirror = 0x141,  // row_half_mirror: lane 7 - i within each 8 lanes
  kDppMirror = 0x140,      // row_mirror: lane 15 - i within each 16 lanes
};

template <int kCtrl>
__device__ __forceinline__ float dpp_read(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of kLanes lanes (kLanes a power of two <= 64);
// every lane of the group receives the same bits (each step adds the same
// two operands in both partner lanes). The whole wavefront must be active.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (kLanes >= 2) v += dpp_read<kDppQuadSwap1>(v);
  if constexpr (kLanes >= 4) v += dpp_read<kDppQuadSwap2>(v);
  if constexpr (kLanes >= 8) v += dpp_read<kDppHalfMirror>(v);
  if constexpr (kLanes >= 16) v += dpp_read<kDppMirror>(v);
  if constexpr (kLanes >= 32) v += __shfl_xor(v, 16);
  if constexpr (kLanes >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- translation
// Block translation: token i of a sequence is in logical block i / B at
// offset i % B; the table row maps the logical block to a physical frame.
// Returns the cache row index (frame * B + offset) of the token, the unit
// in which [NB, B, H, D] caches are addressed before head and element.
// The frame is clamped into [0, num_blocks) so a corrupt table entry cannot
// address memory outside the cache.
__device__ __forceinline__ int64_t token_row(const int32_t* table_row, int32_t i, int32_t B,
                                             int64_t num_blocks) {
  const int32_t blk = i / B;
  const int32_t off = i - blk * B;
  const uint32_t frame = min(static_cast<uint32_t>(table_row[blk]),
                             static_cast<uint32_t>(num_blocks - 1));  // num_blocks <= 2^31
  return static_cast<int64_t>(frame) * B + off;
}

}  // namespace pa

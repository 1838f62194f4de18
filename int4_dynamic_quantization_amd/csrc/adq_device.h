// Device helpers shared by the row, split-row and generic kernels:
// 16-bit <-> fp32 conversion, wavefront reductions, and the quantize/pack
// step.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adq_internal.h"

namespace adq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, 32-bit
// data format word).  Lanes whose offset lies past `bytes` read 0 and
// their stores are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Start of row `row` of a tensor with `row_bytes` bytes per row.
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, uint32_t row_bytes) {
  return static_cast<const char*>(base) + row * (int64_t)row_bytes;
}
__device__ __forceinline__ void* row_ptr(void* base, int64_t row, uint32_t row_bytes) {
  return static_cast<char*>(base) + row * (int64_t)row_bytes;
}

// Cache policy bits of streamed (read-once / write-once) buffer accesses:
// 2 = non-temporal (measured 2-9% faster than cached accesses on the row
// kernel; the sc0 / sc1 combinations measured the same within noise).
constexpr int kStreamLoad = 2;
constexpr int kStreamStore = 2;
// sc1 (no nt) on the stores of row-kernel launches that move at most a few
// hundred MB (the planner's threshold, with its measurements, is in the host
// layer): 4096 x 4096 bf16 (117 MB) 24.6 -> 22.7 us, while launches of 1 GB
// and more run 2-4% slower with it than with nt stores.
constexpr int kWriteThroughStore = 16;

// Two packed 16-bit values (element 0 in the low half) -> two floats.
template <int E>
__device__ __forceinline__ f32x2 widen2(uint32_t w) {
  if constexpr (E == kBF16) {
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
}

// Two floats -> two packed 16-bit values, round to nearest even
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950; fp16 overflow -> inf).
template <int E>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
  if constexpr (E == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
  }
}

template <int E>
__device__ __forceinline__ float widen1(uint16_t h) {
  if constexpr (E == kBF16) {
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

template <int E>
__device__ __forceinline__ uint16_t narrow1(float f) {
  return (uint16_t)(narrow2<E>(f, 0.0f) & 0xFFFFu);
}

// 1.0 in both halves of a 32-bit word.
template <int E>
constexpr uint32_t kOnePair = E == kBF16 ? 0x3F803F80u : 0x3C003C00u;

// ---- wavefront reductions (DPP inside each 16-lane row, readlane across rows)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Sum over the 64 lanes; the same value (and the same bits) in every lane.
// Order: butterflies within rows of 16, then (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)),
               fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

// ---- quantization

// 1.5 * 2^23.  For |v| < 2^22, v + kMagic rounded to float lands on an
// integer (spacing 1 in [2^23, 2^24)), chosen round-half-to-even, and the
// float's low mantissa bits hold round(v) in two's complement.  With an
// fma the rounding applies to the exact product a * inv.
constexpr float kMagic = 12582912.0f;

__device__ __forceinline__ uint32_t code_bits(float a, float inv) {
  return __float_as_uint(__builtin_fmaf(a, inv, kMagic));
}

// Low bytes of four words -> one word (byte i from word i).
__device__ __forceinline__ uint32_t gather4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Eight INT8 codes -> two words, column order.
__device__ __forceinline__ u32x2 pack_int8x8(const uint32_t (&q)[8]) {
  return u32x2{gather4(q[0], q[1], q[2], q[3]), gather4(q[4], q[5], q[6], q[7])};
}

// Eight INT4 codes -> one word: byte j holds column 2j in its low nibble
// and column 2j+1 in its high nibble.
__device__ __forceinline__ uint32_t pack_int4x8(const uint32_t (&q)[8]) {
  const uint32_t even = gather4(q[0], q[2], q[4], q[6]);
  const uint32_t odd = gather4(q[1], q[3], q[5], q[7]);
  return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

template <int Q>
constexpr float kQMax = Q == kQInt4 ? 7.0f : 127.0f;

// scale = row max / Q (correctly rounded); inv = v_rcp_f32(scale), within
// 1 ulp of 1/scale and exact for powers of two; 0 for an all-zero row.
// When 1/scale overflows (scale below about 2^-128) the quantizer inputs
// and the scale are both multiplied by boost = 2^64 (exact) before the
// reciprocal, so one fma per code serves every row.
struct RowScale {
  float scale;
  float inv;
  float boost;  // 1, or 2^64 for rows with a tiny scale
};

template <int Q>
__device__ __forceinline__ RowScale row_scale(float m) {
  RowScale r;
  r.scale = m / kQMax<Q>;
  r.boost = 1.0f;
  r.inv = 0.0f;
  if (r.scale > 0.0f) {
    r.inv = __builtin_amdgcn_rcpf(r.scale);
    if (!(r.inv <= 3.4028234e38f)) {
      r.boost = 18446744073709551616.0f;  // 2^64
      r.inv = __builtin_amdgcn_rcpf(r.scale * r.boost);
    }
  }
  return r;
}

// Scales a row's quantizer inputs by rs.boost (register-only; taken for
// rows with a tiny scale).
template <int N>
__device__ __forceinline__ void apply_boost(float (&in)[N], const RowScale& rs) {
  if (rs.boost != 1.0f) {
#pragma unroll
    for (int e = 0; e < N; ++e) in[e] *= rs.boost;
  }
}

}  // namespace adq

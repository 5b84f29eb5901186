// Device helpers shared by the gfx950 attention kernels: element types,
// bf16 packing, wave64 cross-lane reductions on DPP, and exp2/log2 on the
// hardware transcendental unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// bfloat16 / IEEE half stored as raw bits (element tags of the 16-bit paths).
struct bf16_t {
  uint16_t bits;
};
struct f16_t {
  uint16_t bits;
};

// The two 16-bit input formats on the matrix cores: operand vectors, the
// element type (float -> element conversion rounds to nearest even), the
// MFMA shapes and dot product the kernels use, all with fp32 accumulation,
// and the conversion from 8-bit E4M3 floats (exact in both formats: E4M3
// spans 2^-9 .. 448 with 3 mantissa bits).
template <typename E>
struct Half16;
template <>
struct Half16<bf16_t> {
  typedef __bf16 elem;
  typedef bf16x2 v2;
  typedef bf16x4 v4;
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x4 mfma16x16x32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16x16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
  // Two E4M3 bytes (the low or high half of w) -> two elements, exactly.
  template <bool HI>
  static __device__ __forceinline__ v2 from_fp8x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  }
};
template <>
struct Half16<f16_t> {
  typedef _Float16 elem;
  typedef f16x2 v2;
  typedef f16x4 v4;
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x4 mfma16x16x32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16x16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
  template <bool HI>
  static __device__ __forceinline__ v2 from_fp8x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// fp32 -> bf16 with round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// DPP moves within a row of 16 lanes.  Control words (GCN/CDNA DPP):
//   quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
//   row_half_mirror = 0x141 (lane i <- 7-i within 8),
//   row_mirror = 0x140 (lane i <- 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return x;
}

// v_permlane32_swap with the same register as both operands returns
// r[0] = (x[0..31], x[0..31]) and r[1] = (x[32..63], x[32..63]), so each lane
// sees its own value and its partner's (lane ^ 32) in r[0], r[1].
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
// Value of lane ^ 32.
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)(__lane_id() < 32 ? r[1] : r[0]));
}

// v_permlane16_swap with the same register as both operands: r[0] holds the
// even 16-lane row of each pair of rows, r[1] the odd one, so each lane sees
// its own value and that of lane ^ 16.
__device__ __forceinline__ float max_rows16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_rows16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Value of lane ^ 16.
__device__ __forceinline__ float swap_rows16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)((__lane_id() & 16) ? r[0] : r[1]));
}

// Maximum / sum over the 64 lanes, in every lane: DPP within rows of 16, then
// the two lane-swap steps above (no LDS round trip).  All 64 lanes active.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return max_halves(max_rows16(x));
}
__device__ __forceinline__ float wave_sum(float x) { return sum_halves(sum_rows16(row16_sum(x))); }

}  // namespace attn

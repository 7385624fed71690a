// Device-side helpers shared by the gfx950 kernels: element traits,
// 16-byte vector access, DPP row reductions and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockSize = 16;   // tokens per physical block
constexpr int kWave = 64;        // CDNA wavefront width

// ---------------------------------------------------------------- traits --
template <int DT> struct Elt;
template <> struct Elt<PKV_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;
};
template <> struct Elt<PKV_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};
template <> struct Elt<PKV_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};
template <> struct Elt<PKV_FP8_E4M3> {
  static constexpr int kBytes = 1;
  static constexpr int kPer16B = 16;
};

// Bit casts through by-value scalars.  clang's __builtin_bit_cast applied
// directly to an element of an ext_vector_type lvalue (v[i]) reads the
// vector's first element whatever i is, so vector elements are always
// passed through these by value.
__device__ __forceinline__ uint32_t bits_of(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float float_of(uint32_t x) { return __builtin_bit_cast(float, x); }

// Widen the e-th element of a 16-byte chunk to float.
template <int DT>
__device__ __forceinline__ float elem_to_float(const u32x4& v, int e);

template <>
__device__ __forceinline__ float elem_to_float<PKV_F32>(const u32x4& v, int e) {
  return float_of(v[e]);
}
template <>
__device__ __forceinline__ float elem_to_float<PKV_F16>(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  uint16_t h = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}
template <>
__device__ __forceinline__ float elem_to_float<PKV_BF16>(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  // a bfloat16 is the upper half of a binary32: placing it there is exact
  uint32_t f = (e & 1) ? (w & 0xffff0000u) : (w << 16);
  return __builtin_bit_cast(float, f);
}
// E4M3 codes widen exactly with the hardware conversion (OCP format on
// gfx950: bias 7, S.1111.111 = NaN); the byte index must be a constant.
template <>
__device__ __forceinline__ float elem_to_float<PKV_FP8_E4M3>(const u32x4& v, int e) {
  const int w = (int)v[e >> 2];
  switch (e & 3) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

// Every element of a 16-byte chunk widened to float; E4M3 codes two at a
// time with the packed hardware conversion (exact).
template <int KT>
__device__ __forceinline__ void widen_chunk(const u32x4& v, float (&f)[Elt<KT>::kPer16B]) {
  if constexpr (KT == PKV_FP8_E4M3) {
    typedef float float2_ __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int word = (int)v[w];
      const float2_ lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const float2_ hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      f[4 * w] = lo.x;
      f[4 * w + 1] = lo.y;
      f[4 * w + 2] = hi.x;
      f[4 * w + 3] = hi.y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < Elt<KT>::kPer16B; ++e) f[e] = elem_to_float<KT>(v, e);
  }
}

// E4M3 code of a float: nearest code, ties to the even mantissa; |x| >=
// 448 (inf included) saturates to +-448; NaN gives 0x7F.  Written from the
// format: below 2^-6 the codes are the multiples of 2^-9 (8 reaching the
// smallest normal), above it (1 + f/8) 2^(E) with E + 7 in the exponent
// field.  frexp and the scalings are exact, rint rounds to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  if (x != x) return 0x7Fu;
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    int e;
    const float m = frexpf(a, &e);  // a = m 2^e, m in [0.5, 1)
    float f8 = rintf((2.f * m - 1.f) * 8.f);
    int E = e - 1;
    if (f8 == 8.f) {
      f8 = 0.f;
      ++E;
    }
    code = (uint32_t)((E + 7) * 8 + (int)f8);
  }
  return code | sign;
}

// Round float to the storage type (nearest-even) and return its bits.
template <int DT> __device__ __forceinline__ uint32_t float_to_bits(float x);
template <> __device__ __forceinline__ uint32_t float_to_bits<PKV_F32>(float x) {
  return __builtin_bit_cast(uint32_t, x);
}
template <> __device__ __forceinline__ uint32_t float_to_bits<PKV_F16>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint32_t float_to_bits<PKV_BF16>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (Elt<DT>::kBytes == 4) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)float_to_bits<DT>(x);
  }
}

// ------------------------------------------------------------ 16-B access --
__device__ __forceinline__ float lane_float(const u32x4& v, int e) { return float_of(v[e]); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming reads.  Data read once per call (a key or value tile) is loaded
// with the non-temporal cache policy, which on gfx950 raises the sustained
// read rate from HBM (16-B reads of a 2-GiB buffer: ~6.3 TB/s plain,
// ~7.1 TB/s non-temporal) but gives up reuse from the cache.  The loads go
// through a raw buffer resource: an intrinsic whose cache policy is an
// operand, so the optimizer cannot merge it with a plain load of the same
// address on another path (which would drop the hint).
constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer descriptor, word 3 (32-bit data)
constexpr int kCacheDefault = 0;          // buffer instruction cache policy: default
constexpr int kCacheNonTemporal = 2;      // buffer instruction cache-policy bit: nt

// `bytes` bytes at `base`; offsets outside [0, bytes) read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferWord3);
}
template <int kPolicy>
__device__ __forceinline__ u32x4 load16_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicy));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ------------------------------------------------------------------ DPP --
// Row = 16 consecutive lanes.  Control codes of the gfx9 DPP encoding.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i in each 8-lane half
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i in each row
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16
constexpr int kDppRowRor4 = 0x124;       // lane i <- lane (i+4) mod 16

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xf, 0xf, false));
}

// Max / sum over the 16 lanes of each row; every lane gets the row result.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  x += dpp_f<kDppRowMirror>(x);
  return x;
}

// Sum of x over the lanes whose index differs from this lane's only in
// bits >= log2(STRIDE) (STRIDE in {4,8,16,32}): lanes that share lane % STRIDE.
template <int STRIDE>
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  if constexpr (STRIDE <= 4) x += dpp_f<kDppRowRor4>(x);
  if constexpr (STRIDE <= 8) x += dpp_f<kDppRowRor8>(x);
  if constexpr (STRIDE <= 16) x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// Max of x over the same lanes as sum_over_lane_groups.
template <int STRIDE>
__device__ __forceinline__ float max_over_lane_groups(float x) {
  if constexpr (STRIDE <= 4) x = fmaxf(x, dpp_f<kDppRowRor4>(x));
  if constexpr (STRIDE <= 8) x = fmaxf(x, dpp_f<kDppRowRor8>(x));
  if constexpr (STRIDE <= 16) x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}

__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ------------------------------------------- matrix-core operand moves --
// Four 16-bit elements of one column from four rows, through the gfx950
// transposing LDS read.  In each group of 16 lanes, lane a + 4e passes the
// address of 4 consecutive elements of row e (columns 4a .. 4a+3); lane
// 4a + b then receives column 4a + b of rows 0..3 (checked on the GPU).
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr16(const char* lds_addr) {
  const short4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(lds_addr));
  return uint2{(uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16),
               (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16)};
}

// The value of lane l ^ 16 and of lane l ^ 32, combined with max / sum
// across the four lanes l, l^16, l^32, l^48 (one row's lanes), through the
// row-swapping permutes.
__device__ __forceinline__ float max4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}
__device__ __forceinline__ float sum4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

// Two floats rounded (nearest-even) to the 16-bit type, packed lo | hi << 16.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == PKV_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)lo, (_Float16)hi});
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2{(__bf16)lo, (__bf16)hi});
  }
}

// One 16x16x32 product of 16-bit operands, float32 accumulation.
template <int DT>
__device__ __forceinline__ floatx4 mfma32(const u32x4& a, const u32x4& b, const floatx4& c) {
  if constexpr (DT == PKV_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Four probabilities as eight k slots of a 16-bit MFMA operand: each
// rounded to the 16-bit type, then the remainder of that rounding (exact
// in float32), also rounded.  With the values repeated in both halves the
// product carries p to about 2^-16 of itself (float16: 2^-22), as a
// float32 product would; one rounding alone would leave 2^-9 (bfloat16).
template <int DT>
__device__ __forceinline__ u32x4 split_probs(const float (&pe)[4]) {
  float hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == PKV_F16) hi[i] = (float)(_Float16)pe[i];
    else hi[i] = (float)(__bf16)pe[i];
    lo[i] = pe[i] - hi[i];
  }
  return u32x4{pack2<DT>(pe[0], pe[1]), pack2<DT>(pe[2], pe[3]), pack2<DT>(lo[0], lo[1]),
               pack2<DT>(lo[2], lo[3])};
}

// Four floats stored as the output type (8 bytes for 16-bit types).
template <int DT>
__device__ __forceinline__ void store4(char* dst, const floatx4& v) {
  if constexpr (DT == PKV_F32) {
    store16(dst, u32x4{bits_of(v[0]), bits_of(v[1]), bits_of(v[2]), bits_of(v[3])});
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{float_to_bits<DT>(v[0]) | (float_to_bits<DT>(v[1]) << 16),
              float_to_bits<DT>(v[2]) | (float_to_bits<DT>(v[3]) << 16)};
  }
}

}  // namespace pkv

// MFMA tile helpers for gfx950 (CDNA4, wave64).
//
// A tile is T x T with T = 32 (v_mfma_f32_32x32x2_f32 / _32x32x16_bf16) or
// T = 16 (v_mfma_f32_16x16x4_f32 / _16x16x32_bf16). The lanes of a wave form
// G = 64 / T groups of T lanes; lane l is "column" l % T of group l / T.
//
// Operand layout (both A [M x K] and B [K x N]): lane l supplies the row
// (A) or column (B) l % T, and KL consecutive k values of group g = l / T,
// where KL = 1 for fp32 and KL = 8 for the 16-bit types (bf16, fp16). A
// contraction is free to
// permute k as long as A and B use the same permutation, so the kernels
// pair each lane's 16-byte vector loads with the k values of several
// instructions.
//
// Accumulator layout: lane l holds column l % T; register r holds row
// acc_row<T>(r, g) = 4*G*(r/4) + 4*g + (r%4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that waits for every vector-memory operation and
// leaves the other counters at "no wait"
constexpr int kVmcntZero = (7 << 4) | (15 << 8);
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16 on a row-major 16-bit tile in LDS: the 16 lanes of a
// group pass the addresses of a 4-row x 16-column patch (lane 4k + m: row k,
// columns 4m..4m+3) and lane i receives column i of the 4 rows (V4: a
// 4-vector of the tile's 16-bit type)
template <typename V4>
__device__ __forceinline__ V4 lds_read_tr16_as(const u16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) u16*)p));
  return __builtin_bit_cast(V4, v);
}
__device__ __forceinline__ bf16x4 lds_read_tr16(const u16* p) { return lds_read_tr16_as<bf16x4>(p); }

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), leaving the result in every lane. permlane16_swap returns, for
// each pair of rows (2k, 2k+1), row 2k twice in its first result and row
// 2k+1 twice in its second; permlane32_swap does the same for the two
// halves. Two swaps and two operations, no LDS traffic; every lane ends
// with the bitwise-identical value.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct bf16_t {};  // tag for the bf16 element type (stored as 16-bit words)
struct f16_t {};   // tag for the IEEE fp16 element type (stored as 16-bit words)

// The 16-bit element types: vector types, RNE rounding from float, the
// 16x16x32 / 32x32x16 MFMAs and the two-term dot product (v_dot2_f32_*).
template <typename E>
struct H16;
template <>
struct H16<bf16_t> {
  typedef __bf16 T;
  typedef bf16x8 V8;
  typedef bf16x4 V4;
  typedef bf16x2 V2;
  static __device__ __forceinline__ T cvt(float x) { return (__bf16)x; }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <>
struct H16<f16_t> {
  typedef _Float16 T;
  typedef f16x8 V8;
  typedef f16x4 V4;
  typedef f16x2 V2;
  static __device__ __forceinline__ T cvt(float x) { return (_Float16)x; }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

template <int T>
struct Acc;
template <>
struct Acc<32> { typedef f32x16 type; };
template <>
struct Acc<16> { typedef f32x4 type; };

template <int T>
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return 4 * (64 / T) * (r / 4) + 4 * g + (r % 4);
}

__device__ __forceinline__ void mma(f32x16& c, float a, float b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, float a, float b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, bf16x8 a, bf16x8 b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, bf16x8 a, bf16x8 b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, f16x8 a, f16x8 b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, f16x8 a, f16x8 b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(u16 x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ u16 bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(u16, h);
}

// element type traits: fp32 (KL = 1, 4 floats per 16-byte load) and bf16
// (KL = 8, one 16-byte load feeds one instruction)
template <typename E>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int VEC = 4;   // elements per 16-byte lane load
  static constexpr int KL = 1;    // k values per lane per instruction
  typedef float storage;
};
template <>
struct Elem<bf16_t> {
  static constexpr int VEC = 8;
  static constexpr int KL = 8;
  typedef u16 storage;
};
template <>
struct Elem<f16_t> {
  static constexpr int VEC = 8;
  static constexpr int KL = 8;
  typedef u16 storage;
};

// 16-byte operand fragment of one lane, as the MFMA wants it
template <typename E>
struct Frag;
template <>
struct Frag<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  // elements p[0], p[s], p[2 s], p[3 s] (an operand stored the other way round)
  __device__ __forceinline__ void load_strided(const float* p, int64_t s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = p[q * s];
  }
  __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
};
template <typename E>
struct Frag16 {
  typename H16<E>::V8 v;
  __device__ __forceinline__ void load(const u16* p) { v = *reinterpret_cast<const typename H16<E>::V8*>(p); }
  // elements p[0], p[s], ..., p[7 s]
  __device__ __forceinline__ void load_strided(const u16* p, int64_t s) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = __builtin_bit_cast(typename H16<E>::T, p[q * s]);
  }
  __device__ __forceinline__ void zero() {
    const typename H16<E>::T z = H16<E>::cvt(0.f);
    v = typename H16<E>::V8{z, z, z, z, z, z, z, z};
  }
};
template <>
struct Frag<bf16_t> : Frag16<bf16_t> {};
template <>
struct Frag<f16_t> : Frag16<f16_t> {};

// acc += A-frag x B-frag over the 16 bytes each lane holds
template <int T>
__device__ __forceinline__ void mma_frag(typename Acc<T>::type& c, const Frag<float>& a, const Frag<float>& b) {
  mma(c, a.v[0], b.v[0]);
  mma(c, a.v[1], b.v[1]);
  mma(c, a.v[2], b.v[2]);
  mma(c, a.v[3], b.v[3]);
}
template <int T>
__device__ __forceinline__ void mma_frag(typename Acc<T>::type& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  mma(c, a.v, b.v);
}
template <int T>
__device__ __forceinline__ void mma_frag(typename Acc<T>::type& c, const Frag<f16_t>& a, const Frag<f16_t>& b) {
  mma(c, a.v, b.v);
}

// store one output element of type E from a float accumulator value
template <typename E>
__device__ __forceinline__ void store_elem(typename Elem<E>::storage* p, float x) {
  if constexpr (std::is_same<E, float>::value) {
    *p = x;
  } else {
    const typename H16<E>::T h = H16<E>::cvt(x);
    *p = __builtin_bit_cast(u16, h);
  }
}

}  // namespace bsa

// Device-side helpers shared by the libpagedattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

template <Dt T>
struct EltBytes {
  static constexpr int value = (T == Dt::F32) ? 4 : 2;
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Two floats -> two packed 16-bit values (lo in bits 0-15), nearest even.
template <bool kBf16>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  if constexpr (kBf16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

// ------------------------------------------------ 16-byte fragment arithmetic
// A fragment is the 16 bytes one lane loads with one global_load_dwordx4:
// 8 fp16/bf16 elements or 4 fp32 elements.

template <Dt T>
struct Frag {
  static constexpr int kElems = 16 / EltBytes<T>::value;
};

// sum_i a_i * b_i over one fragment, in fp32.
template <Dt T>
__device__ __forceinline__ float frag_dot(const uint4 &a, const uint4 &b) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
  if constexpr (T == Dt::F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, av[i]), __builtin_bit_cast(half2_t, bv[i]), s,
                                 false);
  } else if constexpr (T == Dt::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, av[i]), __builtin_bit_cast(bf162_t, bv[i]),
                                          s, false);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(av[i]), __uint_as_float(bv[i]), s);
  }
  return s;
}

// acc[e] += p * v[e] for the elements of one fragment.
template <Dt T>
__device__ __forceinline__ void frag_axpy(float *acc, float p, const uint4 &v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (T == Dt::F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h = __builtin_bit_cast(half2_t, w[i]);
      acc[2 * i] = fmaf(p, (float)h.x, acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, (float)h.y, acc[2 * i + 1]);
    }
  } else if constexpr (T == Dt::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(p, bf16_lo(w[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, bf16_hi(w[i]), acc[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(p, __uint_as_float(w[i]), acc[i]);
  }
}

// Store kElems floats as one fragment of type T.
template <Dt T>
__device__ __forceinline__ uint4 frag_pack(const float *x) {
  uint32_t w[4];
  if constexpr (T == Dt::F16 || T == Dt::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_pair<T == Dt::BF16>(x[2 * i], x[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------- K/V rows on wave lanes
// The K (or V) row of one token and head is D elements, D*elt contiguous
// bytes in the cache.  The decode-style kernels cover a row with kLPT
// lanes doing one 16-byte load each, so one wave load covers kGroups
// consecutive tokens and a tile of kTile tokens takes kNI loads.
template <Dt T, int D, int kTile>
struct RowShape {
  static constexpr int kEB = EltBytes<T>::value;
  static constexpr int kRowBytes = D * kEB;         // one token row of one head
  static constexpr int kLPT = kRowBytes / 16;       // lanes per token row
  static constexpr int kGroups = kWave / kLPT;      // tokens per wave load
  static constexpr int kNI = kTile / kGroups;       // loads per tile
  static constexpr int kFE = Frag<T>::kElems;       // elements per lane fragment
  static_assert(kRowBytes % 16 == 0 && kLPT >= 1 && kLPT <= kWave, "row must be whole fragments");
  static_assert(kTile % kGroups == 0, "tile must be whole wave loads");
  static_assert(kLPT * kFE == D, "fragments must tile the head");
};

// 16 bytes, non-temporal: K/V bytes that a launch reads exactly once.
__device__ __forceinline__ uint4 load_nt16(const char *p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------ lane exchange
// DPP controls (GCN/CDNA encoding): quad_perm [1,0,3,2] and [2,3,0,1],
// row_half_mirror (lane i of an 8-lane half-row reads lane 7-i), row_mirror
// (lane i of a 16-lane row reads lane 15-i).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G in 1..64, power of two); every lane
// of a group ends with the group total.  Within a 16-lane row the pairings
// xor1, xor2, xor7 (half mirror) and xor15 (mirror) generate every lane of
// the row, so four DPP adds reduce 16 lanes; wider groups add lane swaps.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<kDppXor1>(x);
  if constexpr (G >= 4) x += dpp<kDppXor2>(x);
  if constexpr (G >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (G >= 16) x += dpp<kDppMirror>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (G >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Read-only kernel input seen through the constant address space: a load at
// a wave-uniform index becomes a scalar (SMEM) load, counted on lgkmcnt, so
// it never waits behind the vector loads in flight.  Only for memory the
// calling kernel does not write.
template <typename T>
__device__ __forceinline__ T load_uniform(const T *p, int64_t i) {
  return ((const __attribute__((address_space(4))) T *)p)[i];
}

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace pa

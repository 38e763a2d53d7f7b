// sq_common.h -- device helpers shared by the gfx950 kernels of libsqw8a8.
// Internal to the library; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace sqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// byte address of a __shared__ object, as LDS instructions take it
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// bf16 halves of a packed 32-bit word, widened exactly to fp32
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Eight consecutive input elements widened to fp32.  bf16: one 16-byte load;
// fp32: two 16-byte loads.  `p` must be 16-byte aligned.
struct Bf16In {
  typedef uint16_t elem;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void load8(const uint16_t* p, float (&o)[8]) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf_lo(v[i]);
      o[2 * i + 1] = bf_hi(v[i]);
    }
  }
  // raw form kept in registers between the load and its use
  struct Raw { u32x4 v; };
  __device__ __forceinline__ static Raw raw8(const uint16_t* p) {
    Raw r;
    r.v = *reinterpret_cast<const u32x4*>(p);
    return r;
  }
  // non-temporal: for data streamed once (the activations into the
  // quantizer, the calibration set), so that it does not push out of the
  // caches what the next kernels read again
  __device__ __forceinline__ static Raw raw8_nt(const uint16_t* p) {
    Raw r;
    r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return r;
  }
  __device__ __forceinline__ static Raw raw8_cached(const uint16_t* p) {
    Raw r;
    r.v = *reinterpret_cast<const u32x4*>(p);
    return r;
  }
  // the first nv (< 8) of the eight elements at p; the rest read as 0 and are
  // not touched in memory (the ragged end of a row)
  __device__ __forceinline__ static Raw raw8_part(const uint16_t* p, int nv) {
    Raw r;
    r.v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nv) r.v[i >> 1] |= (uint32_t)p[i] << (16 * (i & 1));
    return r;
  }
  // hide the value from the optimizer, so that values derived from it are
  // recomputed rather than kept alive
  __device__ __forceinline__ static void opaque(Raw& r) { asm volatile("" : "+v"(r.v)); }
  __device__ __forceinline__ static void widen(const Raw& r, float (&o)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf_lo(r.v[i]);
      o[2 * i + 1] = bf_hi(r.v[i]);
    }
  }
};

struct F32In {
  typedef float elem;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static void load8(const float* p, float (&o)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = a[i];
      o[4 + i] = b[i];
    }
  }
  struct Raw { f32x4 a, b; };
  __device__ __forceinline__ static Raw raw8(const float* p) {
    Raw r;
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
    return r;
  }
  __device__ __forceinline__ static Raw raw8_nt(const float* p) {
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    return r;
  }
  __device__ __forceinline__ static Raw raw8_cached(const float* p) {
    Raw r;
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
    return r;
  }
  __device__ __forceinline__ static Raw raw8_part(const float* p, int nv) {
    Raw r;
    r.a = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    r.b = r.a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nv) r.a[i] = p[i];
      if (i + 4 < nv) r.b[i] = p[i + 4];
    }
    return r;
  }
  __device__ __forceinline__ static void opaque(Raw& r) {
    asm volatile("" : "+v"(r.a));
    asm volatile("" : "+v"(r.b));
  }
  __device__ __forceinline__ static void widen(const Raw& r, float (&o)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = r.a[i];
      o[4 + i] = r.b[i];
    }
  }
};

// Eight consecutive elements at p of which nv exist (nv >= 8: all of them,
// one or two 16-byte loads; else the first nv, the rest 0).
template <class In>
__device__ __forceinline__ typename In::Raw raw8_upto(const typename In::elem* p, int64_t nv) {
  return nv >= 8 ? In::raw8(p) : In::raw8_part(p, (int)nv);
}

// Butterfly reductions across the 64 lanes of a wave.  The combining order is
// fixed, so the result is deterministic.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Non-negative floats order like their bit patterns, so a float maximum of
// values >= +0 is an unsigned integer maximum.
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// Rounding by the reciprocal.  For a step d > 0 with rc = fp32(1/d) finite and
// a quotient below 128 in magnitude, y = fp32(v * rc) lies within 2.3e-5 of
// the correctly rounded quotient fp32(v / d): when y is farther than 2^-15
// from every half-integer, both round to the same integer.  A distance
// |y - rint(y)| above kTieBand marks the values that must be redone with the
// IEEE division.
constexpr float kTieBand = 0.5f - 0x1p-15f;

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  uint16_t ua = __builtin_bit_cast(uint16_t, a);
  uint16_t ub = __builtin_bit_cast(uint16_t, b);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// Symmetric INT8 code of a quotient that is already an integer-valued float
// in [-127, 127]: the low byte of the two's-complement integer.
__device__ __forceinline__ uint32_t code_byte(float r) {
  return (uint32_t)((int)r) & 0xffu;
}

}  // namespace sqk

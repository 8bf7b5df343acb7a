// Device-side helpers shared by libsgmv's kernels (gfx950): packed 16-bit element
// access, 16-byte vector loads and the MFMA 16x16x32 wrappers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/sgmv.h"

namespace sgmv_dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// ------------------------------------------------------------------------------------
// the workspace's flag word (its first int32): bits set by device-side checks, never
// cleared by a kernel (sgmv_check_workspace reads and clears them)
// ------------------------------------------------------------------------------------
constexpr int32_t kFlagWaitTimeout = SGMV_FLAG_WAIT_TIMEOUT;
constexpr int32_t kFlagBadId = SGMV_FLAG_ADAPTER_ID;
constexpr int32_t kFlagSegBounds = SGMV_FLAG_SEG_BOUNDS;

__device__ inline void raise_flag(int32_t* flag, int32_t bit) {
  __hip_atomic_fetch_or(flag, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------
// element helpers: 16-bit values travel packed two per 32-bit word
// ------------------------------------------------------------------------------------
template <int DT>
struct Elem;

template <>
struct Elem<SGMV_F16> {
  static __device__ inline float lo(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
  }
  static __device__ inline float hi(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
  }
  static __device__ inline uint32_t pack(float a, float b) {
    const uint32_t ua = __builtin_bit_cast(uint16_t, static_cast<_Float16>(a));
    const uint32_t ub = __builtin_bit_cast(uint16_t, static_cast<_Float16>(b));
    return ua | (ub << 16);
  }
  static __device__ inline f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Elem<SGMV_BF16> {
  static __device__ inline float lo(uint32_t u) { return __uint_as_float(u << 16); }
  static __device__ inline float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
  static __device__ inline uint32_t pack(float a, float b) {
    const uint32_t ua = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
    const uint32_t ub = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
    return ua | (ub << 16);
  }
  static __device__ inline f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

// Global-memory pointers.  A pointer read out of a device table (the per-segment weight
// pointers) or kept in a private array is generic to the compiler, which then emits flat
// accesses; those count against both the vector-memory and the LDS/scalar wait counters,
// so every wait on them drains all loads in flight.  Casting to address space 1 keeps
// them global loads with exact wait counts.
template <typename T>
using gptr = T __attribute__((address_space(1)))*;
template <typename T>
__device__ inline gptr<const T> global_ptr(const T* p) { return (gptr<const T>)p; }
template <typename T>
__device__ inline gptr<T> global_ptr(T* p) { return (gptr<T>)p; }

__device__ inline uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline uint4 ld16(gptr<const uint16_t> p) {
  const u32x4_t v = *(gptr<const u32x4_t>)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// NW consecutive 32-bit words at p (p aligned to 4*NW bytes), as one vector access
template <int NW>
__device__ inline void load_words(const uint16_t* p, uint32_t* out) {
  if constexpr (NW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x; out[1] = v.y;
  } else {
    out[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int NW>
__device__ inline void store_words(uint16_t* p, const uint32_t* in) {
  if constexpr (NW == 4) {
    *reinterpret_cast<uint4*>(p) = make_uint4(in[0], in[1], in[2], in[3]);
  } else if constexpr (NW == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(in[0], in[1]);
  } else {
    *reinterpret_cast<uint32_t*>(p) = in[0];
  }
}

template <int NW>
__device__ inline void load_words(gptr<const uint16_t> p, uint32_t* out) {
  if constexpr (NW == 4) {
    const u32x4_t v = *(gptr<const u32x4_t>)p;
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else if constexpr (NW == 2) {
    const u32x2_t v = *(gptr<const u32x2_t>)p;
    out[0] = v.x; out[1] = v.y;
  } else {
    out[0] = *(gptr<const uint32_t>)p;
  }
}

template <int NW>
__device__ inline void store_words(gptr<uint16_t> p, const uint32_t* in) {
  if constexpr (NW == 4) {
    *(gptr<u32x4_t>)p = u32x4_t{in[0], in[1], in[2], in[3]};
  } else if constexpr (NW == 2) {
    *(gptr<u32x2_t>)p = u32x2_t{in[0], in[1]};
  } else {
    *(gptr<uint32_t>)p = in[0];
  }
}

__device__ inline uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// element e (0..7) of a 16-byte vector of 16-bit values, as float
template <int DT>
__device__ inline float elem(const uint4& v, int e) {
  const uint32_t w = word(v, e >> 1);
  return (e & 1) ? Elem<DT>::hi(w) : Elem<DT>::lo(w);
}

// sum of the 8 products of two 16-byte vectors, in a fixed order, added to acc
template <int DT>
__device__ inline float dot8(const uint4& a, const uint4& b, float acc) {
  using E = Elem<DT>;
  acc = fmaf(E::lo(a.x), E::lo(b.x), acc);
  acc = fmaf(E::hi(a.x), E::hi(b.x), acc);
  acc = fmaf(E::lo(a.y), E::lo(b.y), acc);
  acc = fmaf(E::hi(a.y), E::hi(b.y), acc);
  acc = fmaf(E::lo(a.z), E::lo(b.z), acc);
  acc = fmaf(E::hi(a.z), E::hi(b.z), acc);
  acc = fmaf(E::lo(a.w), E::lo(b.w), acc);
  acc = fmaf(E::hi(a.w), E::hi(b.w), acc);
  return acc;
}

// Sum of ks float slices src[0], src[stride], ... in the one order every table-path kernel
// uses for split-K slices: four partial sums p_q over slices q, q + 4, q + 8, ... (in
// increasing slice order), then ((p0 + p1) + (p2 + p3)) + 0.  reduce_v_kernel starts each
// p_q from +0 instead; the two differ at most in the sign of a zero along the way, which
// the final + 0 removes, so both give the same bits.  8 loads in flight.
__device__ inline float sum_slices(const float* __restrict__ src, int64_t stride, int ks) {
  float p[4];
  for (int k0 = 0; k0 < ks; k0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (k0 + u < ks) ? src[(k0 + u) * stride] : 0.f;
    if (k0 == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = v[q] + v[q + 4];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u & 3] += v[u];
    }
  }
  return ks > 0 ? ((p[0] + p[1]) + (p[2] + p[3])) + 0.f : 0.f;
}

// Fourth word of a raw buffer resource on gfx950 (32-bit data format, no swizzle, no
// stride): offsets are in bytes and accesses at or past num_records are dropped.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache-policy operand of the buffer-store builtins on gfx950: sc1, a device-scope store,
// which the L2 writes through instead of keeping the line dirty until the write-back at
// the kernel's end.
constexpr int kStoreSc1 = 16;

}  // namespace sgmv_dev

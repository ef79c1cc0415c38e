// Device helpers shared by the libgdn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- dtypes ---

struct f32_t {};   // tag: fp32 storage
struct bf16_t {};  // tag: bf16 storage (raw uint16 bits in memory)

template <typename T> struct io;
template <> struct io<f32_t> {
  using storage = float;
  static constexpr int bytes = 4;
  __device__ static inline float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void store(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};
template <> struct io<bf16_t> {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  __device__ static inline float load(const void* p, int64_t i) {
    uint32_t u = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(u << 16);
  }
  __device__ static inline void store(void* p, int64_t i, float x) {
    __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
    static_cast<__bf16*>(p)[i] = h;
  }
};

__device__ inline float bf16_bits_to_float(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// beta / log-alpha element i of a gate array stored in bf16 or fp32.
__device__ inline float load_gate(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_bits_to_float(static_cast<const uint16_t*>(p)[i])
              : static_cast<const float*>(p)[i];
}

// ------------------------------------------------------------ reductions ---

__device__ inline float wave_sum_xor(float x, int lane_mask) {
  // butterfly over the lanes selected by lane_mask bits (powers of two)
  for (int m = 32; m >= 1; m >>= 1)
    if (lane_mask & m) x += __shfl_xor(x, m, 64);
  return x;
}

// ------------------------------------------------------------------ MFMA ---
// One 16x16 output tile, K = 32 per call.  Lane l holds, for A, row l%16 and
// the eight K-slots 8*(l/16) .. 8*(l/16)+7; for B, column l%16 and the same
// K-slots; the accumulator holds column l%16, rows 4*(l/16) .. +3.  Which
// actual K index a slot stands for is up to the caller, as long as A and B
// use the same assignment.

__device__ inline floatx4 mma32(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 operands: eight 16x16x4 products.  Product j takes slot j of every
// lane group, so each K index is used exactly once.
__device__ inline floatx4 mma32(const floatx8& a, const floatx8& b, floatx4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

template <typename T> struct frag;
template <> struct frag<bf16_t> {
  using type = bf16x8;
  __device__ static inline type from_floats(const float* x) {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
    return r;
  }
  __device__ static inline type zero() {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)0.0f;
    return r;
  }
};
template <> struct frag<f32_t> {
  using type = floatx8;
  __device__ static inline type from_floats(const float* x) {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = x[i];
    return r;
  }
  __device__ static inline type zero() {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0.0f;
    return r;
  }
};

}  // namespace gdn

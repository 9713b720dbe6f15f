// Device helpers shared by the layer's HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; inputs are finite.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Exact GELU, 0.5 z (1 + erf(z / sqrt 2)), with the device erff.
__device__ __forceinline__ float gelu_exact(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
}

// SiLU(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (each about
// 1 ulp): 4 instructions instead of the ~25 of expf and an IEEE division. The
// relative error stays near 1e-7, far below the bfloat16 rounding of the
// hidden activation and within the float32 layer tolerance. For z below about
// -88 the exponential overflows to +inf and the result is -0 (exact: ~-z e^z).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// Rows [*beg, *end) of expert e that its FFN processes: at most `cap` rows
// (the expert's capacity; the grouping is stable, so these are its first cap
// tokens in token order), clamped into [0, S): offsets that do not describe a
// grouping of S rows give wrong results but never an access outside the
// S-row buffers.
__device__ __forceinline__ void expert_rows(const int32_t* __restrict__ offsets, int e, int S, int cap,
                                            int* beg, int* end) {
  const int b = min(max(offsets[e], 0), S);
  const int n = min(max(offsets[e + 1], b), S) - b;
  *beg = b;
  *end = b + min(n, cap);  // cap may be INT_MAX: never form b + cap
}

// Which expert owns global m-tile `mt` when every expert's rows are cut into
// tiles of `bm` rows. Returns false if `mt` is past the last tile.
// offsets: [E+1] exclusive prefix of the per-expert row counts (clamped to [0, S));
// each expert contributes at most cap rows.
__device__ __forceinline__ bool find_m_tile(const int32_t* __restrict__ offsets, int E, int S, int cap,
                                            int bm, int mt, int* expert, int* row0, int* rows) {
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    int beg, end;
    expert_rows(offsets, e, S, cap, &beg, &end);
    const int cnt = end - beg;
    const int nt = (cnt + bm - 1) / bm;
    if (mt < acc + nt) {
      const int local = mt - acc;
      *expert = e;
      *row0 = beg + local * bm;
      *rows = min(bm, cnt - local * bm);
      return true;
    }
    acc += nt;
  }
  return false;
}

}  // namespace moe

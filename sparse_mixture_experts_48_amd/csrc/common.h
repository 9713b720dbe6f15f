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

// Ragged m-tiles: every expert's rows (at most cap of them) are cut into tiles
// of `bm` rows, experts in index order.
// The enumeration is done by one wave at once (E <= 64; every lane of the
// wave must be active): lane e holds expert e's row range and tile count, a
// prefix sum over the lanes gives every expert's first tile, and a ballot finds
// the owner of a tile. One round of loads instead of a serial scan over E.
struct WaveTiles {
  int beg, cnt, incl;  // this lane's expert: first row, rows, tiles up to and including it
  int total;           // m-tiles over all experts (wave-uniform)
};

// ks > 1: an expert whose last m-tile holds at most tail_max rows (a short
// tail) has that tile split into ks tiles, each over one part of the reduction.
__device__ __forceinline__ int expert_mtiles(int cnt, int bm, int ks, int tail_max) {
  const int rem = cnt % bm;
  return (cnt + bm - 1) / bm + ((ks > 1 && rem > 0 && rem <= tail_max) ? ks - 1 : 0);
}

__device__ __forceinline__ WaveTiles wave_tiles(const int32_t* __restrict__ offsets, int E, int S, int cap,
                                                int bm, int ks = 1, int tail_max = 0) {
  const int lane = static_cast<int>(threadIdx.x % 64);
  WaveTiles w{0, 0, 0, 0};
  int nt = 0;
  if (lane < E) {
    int b, e;
    expert_rows(offsets, lane, S, cap, &b, &e);
    w.beg = b;
    w.cnt = e - b;
    nt = expert_mtiles(w.cnt, bm, ks, tail_max);
  }
  int incl = nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  w.incl = incl;
  w.total = __shfl(incl, 63);
  return w;
}

// Owner of m-tile mt (wave-uniform, 0 <= mt < w.total). With split tails
// (ks > 1, as passed to wave_tiles), *split is the part of the reduction a
// tile of a split tail takes (0 .. ks-1), and -1 for every other tile.
__device__ __forceinline__ void wave_tile_owner(const WaveTiles& w, int bm, int mt, int* expert, int* row0,
                                                int* rows, int ks = 1, int tail_max = 0, int* split = nullptr) {
  // tile counts are non-negative, so the lanes whose tiles all lie at or
  // before mt form a prefix of the wave
  const int e = __popcll(__ballot(w.incl <= mt));
  const int cnt = __shfl(w.cnt, e);
  const int first = __shfl(w.incl, e) - expert_mtiles(cnt, bm, ks, tail_max);
  int local = mt - first;
  const int full = cnt / bm;
  int sp = -1;
  if (ks > 1 && local >= full && cnt % bm > 0 && cnt % bm <= tail_max) {
    sp = local - full;
    local = full;
  }
  *expert = e;
  *row0 = __shfl(w.beg, e) + local * bm;
  *rows = min(bm, cnt - local * bm);
  if (split != nullptr) *split = sp;
}

}  // namespace moe

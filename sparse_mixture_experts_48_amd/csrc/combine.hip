// Gated combine: y[t] = sum_j gate[t][j] * o_perm[token_slot[t][j]], over the
// slots that were not dropped (token_slot = -1; Lensa ML explainer "Mixture of
// Experts", Step 5: a token whose every slot is dropped gets 0 from the layer).
//
// maptheai.com "Mixture of Experts", section "The mechanism": the chosen
// experts' outputs are added, weighted by the router's scores; Lensa ML
// explainer "Mixture of Experts", Step 3: y = sum g * E(h).
//
// A gather, not a scatter: every y element has exactly one writer, the K terms
// are accumulated in float32 in ascending j with fmaf, and rounded once, so
// the result does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCombThreads = 256;
constexpr int kCombMaxK = 8;

// Four outputs of one row: one 16-byte (float) or 8-byte (bfloat16) store.
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// Block (t, part): token t (blockIdx.x), float4 columns part*256 + thread. The
// token's slots and gates are the same for the whole block; all K rows are
// loaded before the first fma.
template <typename Tout>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float* __restrict__ o_perm,
                                                               const int32_t* __restrict__ token_slot,
                                                               const float* __restrict__ gate, int T, int d, int K,
                                                               Tout* __restrict__ y) {
  const int t = blockIdx.x;
  const int c4 = blockIdx.y * kCombThreads + threadIdx.x;
  if (c4 >= d / 4) return;
  int s[kCombMaxK];
  float g[kCombMaxK];
  float4 o[kCombMaxK];
#pragma unroll
  for (int j = 0; j < kCombMaxK; ++j) {
    s[j] = -1;
    g[j] = 0.0f;
    if (j < K) {
      const int s_raw = token_slot[static_cast<size_t>(t) * K + j];
      // a slot dropped at its expert's capacity (-1) adds nothing; others stay inside o_perm
      s[j] = s_raw < 0 ? -1 : min(s_raw, T * K - 1);
      g[j] = gate[static_cast<size_t>(t) * K + j];
    }
  }
#pragma unroll
  for (int j = 0; j < kCombMaxK; ++j)
    if (s[j] >= 0) o[j] = *reinterpret_cast<const float4*>(o_perm + static_cast<size_t>(s[j]) * d + 4 * c4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kCombMaxK; ++j) {
    if (s[j] >= 0) {
      acc.x = fmaf(g[j], o[j].x, acc.x);
      acc.y = fmaf(g[j], o[j].y, acc.y);
      acc.z = fmaf(g[j], o[j].z, acc.z);
      acc.w = fmaf(g[j], o[j].w, acc.w);
    }
  }
  store4(y + static_cast<size_t>(t) * d + 4 * c4, acc);
}

}  // namespace

hipError_t launch_combine(const float* o_perm, const int32_t* token_slot, const float* topk_gate, int T,
                          int d, int K, bool bf16, void* y, hipStream_t st) {
  if (K < 1 || K > kCombMaxK || d % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>((d / 4 + kCombThreads - 1) / kCombThreads));
  if (bf16) {
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(kCombThreads), 0, st, o_perm, token_slot, topk_gate,
                       T, d, K, static_cast<bf16_t*>(y));
  } else {
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kCombThreads), 0, st, o_perm, token_slot, topk_gate,
                       T, d, K, static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe

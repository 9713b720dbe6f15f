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

template <typename Tout>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_perm,
                                                      const int32_t* __restrict__ token_slot,
                                                      const float* __restrict__ gate, int T, int d, int K,
                                                      Tout* __restrict__ y) {
  const int d4 = d / 4;
  const size_t total = static_cast<size_t>(T) * d4;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(i / d4);
    const int c = static_cast<int>(i % d4) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < K; ++j) {
      const int s_raw = token_slot[static_cast<size_t>(t) * K + j];
      if (s_raw < 0) continue;  // a slot dropped at its expert's capacity adds nothing
      const int s = min(s_raw, T * K - 1);  // stay inside o_perm
      const float g = gate[static_cast<size_t>(t) * K + j];
      const float4 o = *reinterpret_cast<const float4*>(o_perm + static_cast<size_t>(s) * d + c);
      acc.x = fmaf(g, o.x, acc.x);
      acc.y = fmaf(g, o.y, acc.y);
      acc.z = fmaf(g, o.z, acc.z);
      acc.w = fmaf(g, o.w, acc.w);
    }
    Tout* dst = y + static_cast<size_t>(t) * d + c;
    Elem<Tout>::store(dst + 0, acc.x);
    Elem<Tout>::store(dst + 1, acc.y);
    Elem<Tout>::store(dst + 2, acc.z);
    Elem<Tout>::store(dst + 3, acc.w);
  }
}

}  // namespace

hipError_t launch_combine(const float* o_perm, const int32_t* token_slot, const float* topk_gate, int T,
                          int d, int K, bool bf16, void* y, hipStream_t st) {
  const size_t total = static_cast<size_t>(T) * (d / 4);
  const size_t blocks = (total + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
  if (bf16) {
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, o_perm, token_slot, topk_gate,
                       T, d, K, static_cast<bf16_t*>(y));
  } else {
    hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(256), 0, st, o_perm, token_slot, topk_gate,
                       T, d, K, static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe

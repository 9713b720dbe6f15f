// Router of the MoE layer: float32 logits, softmax, top-K, gates, and the
// per-block partial statistics behind the expert counts and the aux loss.
//
// Lensa ML explainer "Mixture of Experts":
//   Step 2 (The Router): logits = h . W_r, then a softmax over the experts.
//   Step 3 (Top-k Routing): keep the K largest; gates are a softmax over the
//     chosen logits (Mixtral), or p_i unrenormalised (Switch top-1).
//   Step 4 (Load Balancing): T*K slots counted per expert; aux = E sum f P.
// Arjun Jaggi, "Mixture of Experts in LLMs", section "Switch Transformers":
//   the router runs in float32.
//
// Numeric contract: each logit is one fmaf chain over k = 0..d-1 from +0,
// bias added afterwards, so the expert choice is independent of any
// parallel-reduction order. A thread owns TPT tokens x TE experts and walks k
// upward; lanes are laid out as [token group][expert lane], so the experts of
// one token sit in LE = EP/TE adjacent lanes of one wave and the per-token
// max / argmax / sum reductions are xor-butterflies inside those lanes.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteBK = 64;           // k values staged in LDS per step
constexpr int kRoutePad = kRouteBK + 4; // row stride in floats (16-byte aligned, bank-skewed)

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <typename Tin> struct Vec8;
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};
template <> struct Vec8<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

template <typename Tin, int EP, int TE, int TPT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const Tin* __restrict__ h, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int d, int E, int K, int gate_mode,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, float* __restrict__ logits_out,
    int32_t* __restrict__ blk_hist, float* __restrict__ blk_psum) {
  constexpr int LE = EP / TE;             // lanes per token
  constexpr int G = kRouteThreads / LE;   // token groups per block
  constexpr int TB = G * TPT;             // tokens per block
  static_assert(LE >= 1 && LE <= 64 && (64 % LE) == 0, "token lanes must tile a wave");

  __shared__ __align__(16) float h_s[TB][kRoutePad];
  __shared__ __align__(16) float w_s[EP][kRoutePad];
  __shared__ float psum_s[G][EP];
  __shared__ int hist_s[EP];

  const int tid = threadIdx.x;
  const int tg = tid / LE;
  const int el = tid % LE;
  const int t0 = blockIdx.x * TB;
  if (tid < EP) hist_s[tid] = 0;

  float acc[TPT][TE];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int q = 0; q < TE; ++q) acc[i][q] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += kRouteBK) {
    const int kn = min(kRouteBK, d - k0);  // a multiple of 8
    // h rows of this block, converted to float32, 8 values per load
    for (int v = tid; v < TB * (kRouteBK / 8); v += kRouteThreads) {
      const int r = v / (kRouteBK / 8);
      const int c = (v % (kRouteBK / 8)) * 8;
      const int t = t0 + r;
      float x[8];
      if (t < T && c < kn) {
        Vec8<Tin>::load(h + static_cast<size_t>(t) * d + k0 + c, x);
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) h_s[r][c + u] = x[u];
    }
    // W_r[k0 .. k0+kn)[0 .. E) transposed into w_s[e][k]
    for (int v = tid; v < kRouteBK * EP; v += kRouteThreads) {
      const int r = v / EP;
      const int c = v % EP;
      float x = 0.0f;
      if (r < kn && c < E) x = Wr[static_cast<size_t>(k0 + r) * E + c];
      w_s[c][r] = x;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; kk += 4) {
      float4 hv[TPT], wv[TE];
#pragma unroll
      for (int i = 0; i < TPT; ++i) hv[i] = *reinterpret_cast<const float4*>(&h_s[tg + i * G][kk]);
#pragma unroll
      for (int q = 0; q < TE; ++q) wv[q] = *reinterpret_cast<const float4*>(&w_s[el * TE + q][kk]);
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int q = 0; q < TE; ++q) {
          acc[i][q] = fmaf(hv[i].x, wv[q].x, acc[i][q]);
          acc[i][q] = fmaf(hv[i].y, wv[q].y, acc[i][q]);
          acc[i][q] = fmaf(hv[i].z, wv[q].z, acc[i][q]);
          acc[i][q] = fmaf(hv[i].w, wv[q].w, acc[i][q]);
        }
    }
    __syncthreads();
  }

  float psum_local[TE];
#pragma unroll
  for (int q = 0; q < TE; ++q) psum_local[q] = 0.0f;

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = t0 + tg + i * G;
    const bool tok_ok = t < T;  // uniform across the LE lanes of this token
    float l[TE];
#pragma unroll
    for (int q = 0; q < TE; ++q) {
      const int e = el * TE + q;
      if (e < E) {
        l[q] = acc[i][q];
        if (br != nullptr) l[q] = l[q] + br[e];
      } else {
        l[q] = -INFINITY;
      }
    }
    if (tok_ok && logits_out != nullptr) {
#pragma unroll
      for (int q = 0; q < TE; ++q) {
        const int e = el * TE + q;
        if (e < E) logits_out[static_cast<size_t>(t) * E + e] = l[q];
      }
    }
    // top-K by (logit descending, expert ascending)
    bool taken[TE];
#pragma unroll
    for (int q = 0; q < TE; ++q) taken[q] = false;
    int cidx[8];
    float cval[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < TE; ++q) {
          const int e = el * TE + q;
          if (!taken[q] && e < E && better(l[q], e, bv, bi)) { bv = l[q]; bi = e; }
        }
#pragma unroll
        for (int off = 1; off < LE; off <<= 1) {
          const float ov = __shfl_xor(bv, off, LE);
          const int oi = __shfl_xor(bi, off, LE);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        cidx[j] = bi;
        cval[j] = bv;
#pragma unroll
        for (int q = 0; q < TE; ++q)
          if (el * TE + q == bi) taken[q] = true;
      }
    }
    // softmax over all E (the largest logit is the first choice)
    const float m = cval[0];
    float ex[TE];
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < TE; ++q) {
      ex[q] = (el * TE + q < E) ? expf(l[q] - m) : 0.0f;
      s += ex[q];
    }
#pragma unroll
    for (int off = 1; off < LE; off <<= 1) s += __shfl_xor(s, off, LE);
    if (tok_ok) {
#pragma unroll
      for (int q = 0; q < TE; ++q) psum_local[q] += ex[q] / s;
    }
    if (tok_ok && el == 0) {
      float ec[8];
      float se = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          ec[j] = expf(cval[j] - m);
          se += ec[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          const float g = (gate_mode == 0) ? ec[j] / se : ec[j] / s;
          topk_idx[static_cast<size_t>(t) * K + j] = cidx[j];
          topk_gate[static_cast<size_t>(t) * K + j] = g;
          atomicAdd(&hist_s[cidx[j]], 1);
        }
      }
    }
  }

#pragma unroll
  for (int q = 0; q < TE; ++q) psum_s[tg][el * TE + q] = psum_local[q];
  __syncthreads();
  if (tid < E) {
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += psum_s[g][tid];
    blk_psum[static_cast<size_t>(blockIdx.x) * E + tid] = s;
    blk_hist[static_cast<size_t>(blockIdx.x) * E + tid] = hist_s[tid];
  }
}

// Per-block expert histogram of topk_idx, with the router's token tiling.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ topk_idx, int T, int E,
                                                   int K, int TB, int32_t* __restrict__ blk_hist) {
  __shared__ int hist_s[64];
  if (threadIdx.x < 64) hist_s[threadIdx.x] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * TB;
  const int t1 = min(T, t0 + TB);
  for (int v = t0 * K + threadIdx.x; v < t1 * K; v += blockDim.x) {
    const int e = topk_idx[v];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist_s[e], 1);  // ignore invalid ids
  }
  __syncthreads();
  if (threadIdx.x < E) blk_hist[static_cast<size_t>(blockIdx.x) * E + threadIdx.x] = hist_s[threadIdx.x];
}

// One block: expert counts, offsets, per-block bases for the stable grouping,
// P_e, and the aux loss. Fixed summation orders only.
constexpr int kFinThreads = 1024;
constexpr int kFinParts = kFinThreads / 64;

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const int32_t* __restrict__ blk_hist, const float* __restrict__ blk_psum, int NB, int T, int E,
    int K, int32_t* __restrict__ blk_base, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, float* __restrict__ prob_mean, float* __restrict__ aux_out) {
  __shared__ int part_cnt[kFinParts][64];
  __shared__ float part_p[kFinParts][64];
  __shared__ int off_s[65];
  __shared__ float P_s[64];
  const int e = threadIdx.x % 64;
  const int part = threadIdx.x / 64;
  const int per = (NB + kFinParts - 1) / kFinParts;
  const int b0 = part * per;
  const int b1 = min(NB, b0 + per);
  int c = 0;
  float ps = 0.0f;
  if (e < E) {
    for (int b = b0; b < b1; ++b) {
      c += blk_hist[static_cast<size_t>(b) * E + e];
      if (blk_psum != nullptr) ps += blk_psum[static_cast<size_t>(b) * E + e];
    }
  }
  part_cnt[part][e] = c;
  part_p[part][e] = ps;
  __syncthreads();
  if (threadIdx.x < 64) {
    int tot = 0;
    float ptot = 0.0f;
    for (int p = 0; p < kFinParts; ++p) {
      tot += part_cnt[p][e];
      ptot += part_p[p][e];
    }
    part_cnt[0][e] = tot;  // reuse row 0 for totals after the read above (same thread)
    P_s[e] = (T > 0) ? ptot / static_cast<float>(T) : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int x = 0; x < E; ++x) {
      off_s[x] = run;
      run += part_cnt[0][x];
    }
    off_s[E] = run;
  }
  __syncthreads();
  if (threadIdx.x < E) {
    if (counts_out != nullptr) counts_out[e] = part_cnt[0][e];
    if (prob_mean != nullptr) prob_mean[e] = P_s[e];
  }
  if (threadIdx.x <= E && offsets_out != nullptr) offsets_out[threadIdx.x] = off_s[threadIdx.x];
  if (threadIdx.x == 0 && aux_out != nullptr) {
    float a = 0.0f;
    const float S = static_cast<float>(T) * static_cast<float>(K);
    for (int x = 0; x < E; ++x) a += (static_cast<float>(part_cnt[0][x]) / S) * P_s[x];
    *aux_out = (T > 0) ? static_cast<float>(E) * a : 0.0f;
  }
  if (blk_base != nullptr) {
    // base[b][e] = offsets[e] + sum_{b' < b} hist[b'][e]; the part prefix is
    // recomputed from blk_hist (part_cnt row 0 now holds totals).
    __syncthreads();
    if (e < E) {
      int pre = off_s[e];
      for (int b = 0; b < b0; ++b) pre += blk_hist[static_cast<size_t>(b) * E + e];
      for (int b = b0; b < b1; ++b) {
        blk_base[static_cast<size_t>(b) * E + e] = pre;
        pre += blk_hist[static_cast<size_t>(b) * E + e];
      }
    }
  }
}

__global__ void zero_outputs_kernel(int E, int32_t* counts, int32_t* offsets, float* prob_mean,
                                    float* aux) {
  const int i = threadIdx.x;
  if (counts != nullptr && i < E) counts[i] = 0;
  if (prob_mean != nullptr && i < E) prob_mean[i] = 0.0f;
  if (offsets != nullptr && i <= E) offsets[i] = 0;
  if (aux != nullptr && i == 0) *aux = 0.0f;
}

template <typename Tin, int EP, int TE>
hipError_t launch_route_tpt(const RouteArgs& a, int tpt, hipStream_t st) {
  const int LE = EP / TE;
  const int G = kRouteThreads / LE;
  const int TB = G * tpt;
  const int nb = (a.T + TB - 1) / TB;
  const Tin* h = static_cast<const Tin*>(a.h);
#define MOE_ROUTE_LAUNCH(TPTV)                                                                    \
  hipLaunchKernelGGL((route_kernel<Tin, EP, TE, TPTV>), dim3(nb), dim3(kRouteThreads), 0, st, h, \
                     a.Wr, a.br, a.T, a.d, a.E, a.K, a.gate, a.topk_idx, a.topk_gate,             \
                     a.logits, a.blk_hist, a.blk_psum)
  switch (tpt) {
    case 1: MOE_ROUTE_LAUNCH(1); break;
    case 2: MOE_ROUTE_LAUNCH(2); break;
    default: MOE_ROUTE_LAUNCH(4); break;
  }
#undef MOE_ROUTE_LAUNCH
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_route_dtype(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  switch (rt.EP) {
    case 8: return launch_route_tpt<Tin, 8, 1>(a, rt.TPT, st);
    case 16: return launch_route_tpt<Tin, 16, 2>(a, rt.TPT, st);
    case 32: return launch_route_tpt<Tin, 32, 2>(a, rt.TPT, st);
    default: return launch_route_tpt<Tin, 64, 4>(a, rt.TPT, st);
  }
}

}  // namespace

RouteTiling route_tiling(int64_t T, int64_t E) {
  RouteTiling rt;
  rt.EP = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
  const int TE = rt.EP == 8 ? 1 : rt.EP == 64 ? 4 : 2;
  const int LE = rt.EP / TE;
  const int G = kRouteThreads / LE;
  // Prefer more tokens per thread (more independent chains, fewer LDS reads
  // per fma) while the grid still has about two blocks per compute unit.
  rt.TPT = 1;
  for (int tpt = 4; tpt >= 2; tpt /= 2) {
    if ((T + G * tpt - 1) / (G * tpt) >= 512) { rt.TPT = tpt; break; }
  }
  rt.TB = G * rt.TPT;
  rt.NB = static_cast<int>((T + rt.TB - 1) / rt.TB);
  return rt;
}

hipError_t launch_route(const RouteArgs& a, const RouteTiling& rt, bool bf16, hipStream_t st) {
  return bf16 ? launch_route_dtype<bf16_t>(a, rt, st) : launch_route_dtype<float>(a, rt, st);
}

hipError_t launch_hist(const int32_t* topk_idx, int T, int E, int K, const RouteTiling& rt,
                       int32_t* blk_hist, hipStream_t st) {
  hipLaunchKernelGGL(hist_kernel, dim3(rt.NB), dim3(256), 0, st, topk_idx, T, E, K, rt.TB, blk_hist);
  return hipGetLastError();
}

hipError_t launch_finalize(const int32_t* blk_hist, const float* blk_psum, int NB, int T, int E, int K,
                           int32_t* blk_base, int32_t* counts, int32_t* offsets, float* prob_mean,
                           float* aux, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kFinThreads), 0, st, blk_hist, blk_psum, NB, T, E,
                     K, blk_base, counts, offsets, prob_mean, aux);
  return hipGetLastError();
}

hipError_t launch_zero_outputs(int E, int32_t* counts, int32_t* offsets, float* prob_mean, float* aux,
                               hipStream_t st) {
  hipLaunchKernelGGL(zero_outputs_kernel, dim3(1), dim3(128), 0, st, E, counts, offsets, prob_mean, aux);
  return hipGetLastError();
}

}  // namespace moe

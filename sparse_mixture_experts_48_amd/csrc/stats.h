// The statistics of the router's per-block partials, formed by one block of
// kFinThreads threads: expert counts, offsets, per-block bases for the stable
// grouping, P_e, the aux loss and the z-loss (Lensa ML explainer "Mixture of
// Experts", Step 4: f_e = count_e / (T K), P_e the mean router probability,
// aux = E sum f P). Fixed summation orders only, so every caller of this
// function gets the same bits. Shared by the finalize kernel and by the
// grouping kernel of a batch small enough for one grouping block.
#pragma once

#include "common.h"

namespace moe {

constexpr int kFinThreads = 1024;
constexpr int kFinParts = kFinThreads / 64;

// Every output is nullable. off_s (shared, E + 1 ints) receives the offsets;
// it is complete when the function returns (all threads of the block call it).
__device__ __forceinline__ void finalize_block(
    const int32_t* __restrict__ blk_hist, const float* __restrict__ blk_psum, const float* __restrict__ blk_z,
    int NB, int T, int E, int K, int32_t* __restrict__ blk_base, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, float* __restrict__ prob_mean, float* __restrict__ aux_out,
    float* __restrict__ z_out, int* off_s) {
  __shared__ int part_cnt[kFinParts][64];
  __shared__ float part_p[kFinParts][64];
  __shared__ float part_z[kFinParts];
  __shared__ int tot_s[64];
  __shared__ float P_s[64];
  const int e = threadIdx.x % 64;
  const int part = threadIdx.x / 64;
  const int per = (NB + kFinParts - 1) / kFinParts;
  const int b0 = min(NB, part * per);
  const int b1 = min(NB, b0 + per);
  // Loads in batches of kU (independent, in flight together), sums in block
  // order. A part of at most kU blocks (NB <= 512) is one batch, and its
  // counts stay in registers for the bases below.
  constexpr int kU = 32;
  int c = 0;
  float ps = 0.0f;
  int hv[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) hv[u] = 0;
  if (e < E) {
    for (int b = b0; b < b1; b += kU) {
      float pv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const bool in = b + u < b1;
        hv[u] = in ? blk_hist[static_cast<size_t>(b + u) * E + e] : 0;
        pv[u] = (in && blk_psum != nullptr) ? blk_psum[static_cast<size_t>(b + u) * E + e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        c += hv[u];
        if (b + u < b1) ps += pv[u];
      }
    }
  }
  part_cnt[part][e] = c;
  part_p[part][e] = ps;
  if (e == 0) {  // z-loss partials of this part's blocks, in block order
    float zs = 0.0f;
    if (blk_z != nullptr) {
      for (int b = b0; b < b1; b += kU) {
        float zv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) zv[u] = (b + u < b1) ? blk_z[b + u] : 0.0f;
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (b + u < b1) zs += zv[u];
      }
    }
    part_z[part] = zs;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int tot = 0;
    float ptot = 0.0f;
    for (int p = 0; p < kFinParts; ++p) {  // fixed order
      tot += part_cnt[p][e];
      ptot += part_p[p][e];
    }
    tot_s[e] = tot;
    P_s[e] = (T > 0) ? ptot / static_cast<float>(T) : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int x = 0; x < E; ++x) {
      off_s[x] = run;
      run += tot_s[x];
    }
    off_s[E] = run;
  }
  __syncthreads();
  if (threadIdx.x < E) {
    if (counts_out != nullptr) counts_out[e] = tot_s[e];
    if (prob_mean != nullptr) prob_mean[e] = P_s[e];
  }
  if (threadIdx.x <= E && offsets_out != nullptr) offsets_out[threadIdx.x] = off_s[threadIdx.x];
  if (threadIdx.x == 0 && z_out != nullptr) {
    float z = 0.0f;
    for (int p = 0; p < kFinParts; ++p) z += part_z[p];  // fixed order
    *z_out = (T > 0) ? z / static_cast<float>(T) : 0.0f;
  }
  if (threadIdx.x == 0 && aux_out != nullptr) {
    float a = 0.0f;
    const float S = static_cast<float>(T) * static_cast<float>(K);
    for (int x = 0; x < E; ++x) a += (static_cast<float>(tot_s[x]) / S) * P_s[x];
    *aux_out = (T > 0) ? static_cast<float>(E) * a : 0.0f;
  }
  if (blk_base != nullptr && e < E) {
    // base[b][e] = offsets[e] + slots of e in blocks before b
    int pre = off_s[e];
    for (int p = 0; p < part; ++p) pre += part_cnt[p][e];
    if (b1 - b0 <= kU) {  // the part's counts are still in hv
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (b0 + u < b1) blk_base[static_cast<size_t>(b0 + u) * E + e] = pre;
        pre += hv[u];
      }
    } else {
      for (int b = b0; b < b1; b += kU) {
#pragma unroll
        for (int u = 0; u < kU; ++u) hv[u] = (b + u < b1) ? blk_hist[static_cast<size_t>(b + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (b + u < b1) blk_base[static_cast<size_t>(b + u) * E + e] = pre;
          pre += hv[u];
        }
      }
    }
  }
}

}  // namespace moe

// Stable grouping of the T*K routing slots by expert.
//
// Lensa ML explainer "Mixture of Experts", Step 5: instead of fixed capacity
// buffers, experts take any number of tokens (dropless). Each expert's rows
// are contiguous; inside a group tokens keep their order, so the result is
// the stable sort of the slots by (expert, token). With a capacity of C slots
// per expert (Step 5), a slot whose rank in its group is C or more is dropped
// (token_slot = -1): each expert keeps its first C tokens in token order.
//
// Block b owns the token ranges of M consecutive router blocks, starting at
// router block b*M (M = 256 / tokens per router block, so a block holds up to
// 256 tokens). Its base row for expert e is that of its first router block,
// offsets[e] + (slots of e in router blocks before it), computed by the
// finalize kernel. Inside the block, wave w takes one round per expert that
// occurs among its 64 tokens: a ballot gives the wave's count, and a token's
// rank is the popcount of the lanes below it that chose the same expert;
// its slot adds the counts of earlier waves.
#include "common.h"
#include "kernels.h"
#include "stats.h"

namespace moe {

namespace {

constexpr int kPermThreads = 256;  // 4 waves x 64 tokens
constexpr int kMaxK = 8;

// FUSED: every grouping block first forms the router statistics itself, as
// the finalize kernel would (the same function, so the same bits), with
// kFinThreads threads; block 0 writes them. Its base row for expert e is then
// offsets[e] plus the slots of e in the router blocks before its own, summed
// over those blocks' histograms. Threads past kPermThreads take part in the
// statistics and in every barrier, and group nothing.
template <bool FUSED>
__global__ __launch_bounds__(FUSED ? kFinThreads : kPermThreads) void permute_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ blk_base,
    const int32_t* __restrict__ offsets, int T, int E, int K, int cap,
    int TB, int M, const char* __restrict__ h, size_t row_bytes, char* __restrict__ h_perm,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ token_slot, FinArgs fin) {
  __shared__ int cnt_s[kPermThreads / 64][64];
  __shared__ int slots_s[kPermThreads][kMaxK];
  __shared__ int base_s[64];
  __shared__ int off_s[65];
  if constexpr (FUSED) {
    const bool first = blockIdx.x == 0;
    finalize_block(fin.blk_hist, fin.blk_psum, fin.blk_z, fin.NB, T, E, K, nullptr, first ? fin.counts : nullptr,
                   first ? fin.offsets : nullptr, first ? fin.prob_mean : nullptr, first ? fin.aux : nullptr,
                   first ? fin.z_loss : nullptr, off_s);
    // slots of each expert in router blocks 0 .. blockIdx.x * M - 1: kFinParts
    // parts of those blocks, one expert per lane, added in part order
    __shared__ int pre_s[kFinParts][64];
    const int e = threadIdx.x % 64, part = threadIdx.x / 64;
    const int nb = min(fin.NB, static_cast<int>(blockIdx.x) * M);
    const int per = (nb + kFinParts - 1) / kFinParts;
    const int b0 = min(nb, part * per), b1 = min(nb, b0 + per);
    int c = 0;
    if (e < E) {
      constexpr int kU = 32;  // loads in flight together
      for (int b = b0; b < b1; b += kU) {
        int hv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) hv[u] = (b + u < b1) ? fin.blk_hist[static_cast<size_t>(b + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kU; ++u) c += hv[u];
      }
    }
    pre_s[part][e] = c;
    __syncthreads();
    if (threadIdx.x < E) {
      int base = off_s[threadIdx.x];
      for (int q = 0; q < kFinParts; ++q) base += pre_s[q][threadIdx.x];
      base_s[threadIdx.x] = base;
    }
  } else {
    if (threadIdx.x < E) {  // one coalesced read instead of one read per expert below
      base_s[threadIdx.x] = blk_base[static_cast<size_t>(blockIdx.x) * M * E + threadIdx.x];
      off_s[threadIdx.x] = offsets[threadIdx.x];
    }
  }
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const bool grp = threadIdx.x < kPermThreads;  // wave-uniform
  const int t0 = blockIdx.x * TB;
  const int lt = threadIdx.x;
  const int t = t0 + lt;
  const bool ok = grp && lt < TB && t < T;
  int ids[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) ids[j] = (ok && j < K) ? topk_idx[static_cast<size_t>(t) * K + j] : -1;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // Pass 1, one round per expert present in the wave (not per expert of the
  // layer): the lanes holding it get their rank among the wave's tokens that
  // chose it (popcount of those below), and the wave's count is recorded.
  // Slot ids outside [0, E) are skipped.
  if (grp) cnt_s[wave][lane] = 0;
  uint32_t rem = 0;  // bit j: slot j of this lane still to rank
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (static_cast<unsigned>(ids[j]) < static_cast<unsigned>(E)) rem |= 1u << j;
  int rk[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) rk[j] = 0;
  for (uint64_t active = __ballot(rem != 0); active != 0; active = __ballot(rem != 0)) {
    const int leader = __builtin_ctzll(active);  // wave-uniform
    int first = -1;
#pragma unroll
    for (int j = kMaxK - 1; j >= 0; --j)
      if ((rem >> j) & 1u) first = ids[j];
    const int e = __builtin_amdgcn_readlane(first, leader);
    uint32_t hit = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (((rem >> j) & 1u) && ids[j] == e) hit |= 1u << j;
    const uint64_t m = __ballot(hit != 0);
    if (lane == 0) cnt_s[wave][e] = __popcll(m);
    const int r = __popcll(m & below);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if ((hit >> j) & 1u) rk[j] = r;
    rem &= ~hit;
  }
  __syncthreads();

  // Pass 2: slot = block base + counts of earlier waves + rank in the wave.
  // A slot id outside [0, E) gets token_slot -1 and no grouped row.
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int e = ids[j];
    if (ok && j < K && static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {
      token_slot[static_cast<size_t>(t) * K + j] = -1;
      slots_s[lt][j] = -1;
    }
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
      int base = base_s[e];
      for (int w = 0; w < wave; ++w) base += cnt_s[w][e];
      const int slot = base + rk[j];
      const bool kept = slot - off_s[e] < cap;  // rank in the expert's group, token order
      token_slot[static_cast<size_t>(t) * K + j] = kept ? slot : -1;
      slots_s[lt][j] = slot;
      slot_token[slot] = t;
    }
  }

  if (h_perm == nullptr) return;
  __syncthreads();
  // Gather: each token row is read once (up to 8 x 16 bytes per lane in flight)
  // and written to its K grouped rows.
  constexpr int kU = 8;
  const int ntok = min(TB, T - t0);
  const int nvec = static_cast<int>(row_bytes / 16);
  for (int r = wave; grp && r < ntok; r += kPermThreads / 64) {
    const uint4* src = reinterpret_cast<const uint4*>(h + static_cast<size_t>(t0 + r) * row_bytes);
    int sl[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) sl[j] = (j < K) ? slots_s[r][j] : 0;
    for (int c0 = 0; c0 < nvec; c0 += 64 * kU) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nvec) v[u] = src[c];
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < K && sl[j] >= 0) {
          uint4* dst = reinterpret_cast<uint4*>(h_perm + static_cast<size_t>(sl[j]) * row_bytes);
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int c = c0 + u * 64 + lane;
            if (c < nvec) dst[c] = v[u];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* topk_idx, const int32_t* blk_base, const int32_t* offsets, int T,
                          int E, int K, int cap, const RouteTiling& rt, const void* h, size_t row_bytes,
                          void* h_perm, int32_t* slot_token, int32_t* token_slot, hipStream_t st) {
  if (rt.TB < 1 || rt.TB > kPermThreads) return hipErrorInvalidValue;
  const int M = kPermThreads / rt.TB;  // router blocks per permute block
  const int nb = (rt.NB + M - 1) / M;
  hipLaunchKernelGGL(permute_kernel<false>, dim3(nb), dim3(kPermThreads), 0, st, topk_idx, blk_base, offsets, T,
                     E, K, cap, M * rt.TB, M, static_cast<const char*>(h), row_bytes, static_cast<char*>(h_perm),
                     slot_token, token_slot, FinArgs{});
  return hipGetLastError();
}

hipError_t launch_finalize_permute(const FinArgs& fin, const int32_t* topk_idx, int T, int E, int K, int cap,
                                   const RouteTiling& rt, const void* h, size_t row_bytes, void* h_perm,
                                   int32_t* slot_token, int32_t* token_slot, hipStream_t st) {
  if (rt.TB < 1 || rt.TB > kPermThreads || fin.NB != rt.NB || fin.blk_hist == nullptr) return hipErrorInvalidValue;
  const int M = kPermThreads / rt.TB;  // router blocks per grouping block
  const int nb = (rt.NB + M - 1) / M;
  hipLaunchKernelGGL(permute_kernel<true>, dim3(nb), dim3(kFinThreads), 0, st, topk_idx, nullptr, nullptr, T, E,
                     K, cap, M * rt.TB, M, static_cast<const char*>(h), row_bytes, static_cast<char*>(h_perm),
                     slot_token, token_slot, fin);
  return hipGetLastError();
}

}  // namespace moe

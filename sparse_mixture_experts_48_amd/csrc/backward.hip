// Backward pass of the MoE layer (bfloat16 layers): the elementwise, gather,
// transpose and reduction kernels around the expert GEMMs.
//
// The gradient reaches the router only through the gate weights of the chosen
// experts (maptheai.com "Mixture of Experts", section "The difficulties": the
// top-k choice is not differentiable) — through p_i for Switch-style gates
// (Lensa ML explainer "Mixture of Experts", Step 3) — and through P of the
// load-balancing loss, whose f is a count (Step 4: only P_i is
// differentiable). The choice and the capacity drops are held fixed.
//
// Loss = sum(dy * y) + daux * aux. With y[t] = sum_j g[t][j] o[slot(t, j)]
// and o[s] = A[s] W2^T + b2:
//   u[s] = dy[t] W2 (rows of W2^T),  dA = g u,  dZ = dA * act'(Z),  dX = dZ [W1; W3]
//   dgate[t][j] = dy[t] . o[s] = A[s] . u[s] + dy[t] . b2
//   (the pre-activation GEMM also writes A = act(Z); the u GEMM forms dA and
//   applies act' in its epilogue, writes dZ and the 64-column partial sums of
//   A . u, so o is never recomputed)
//   dO[s] = g dy[t] (for dW2)
//   dh[t] = sum_j dX[slot(t, j)] + dlogits[t] W_r^T
//   dW2_e = dO_e^T A_e,  dW1_e = dZ1_e^T X_e,  dW3_e = dZ3_e^T X_e
//   dW_r = h^T dlogits,  db_r = sum_t dlogits   (not when the bias only steers the choice)
// The u and dX GEMMs read W2 and [W1; W3] as stored for the forward pass,
// with k as the row index (transposed in the LDS fragment reads). Weight
// gradients need sums over each expert's grouped rows; the rows of the
// operands are transposed into [feature][slot] matrices in which every
// expert's slots start at a multiple of 64 and are padded with zeros to a
// whole number of GEMM stages.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTile = 64;

// Rows each expert keeps, and its padded column range kofs[e] .. kofs[e+1].
__global__ void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int S, int cap,
                                   int32_t* __restrict__ kofs) {
  if (threadIdx.x != 0) return;
  int run = 0;
  for (int e = 0; e < E; ++e) {
    int beg, end;
    expert_rows(offsets, e, S, cap, &beg, &end);
    kofs[e] = run;
    run += (end - beg + kTile - 1) / kTile * kTile;
  }
  kofs[E] = run;
}

// The transpose moves 64 x 64 tiles through LDS in 16-byte pieces: a thread
// loads two runs of 8 elements along a source row and stores two runs of 8
// along a destination row (every row length and offset is a multiple of 8).
constexpr int kTP = kTile + 8;  // LDS row stride of a tile (elements)

// Tile column j <- source row r (8 elements at column f8 of the tile row).
__device__ __forceinline__ void tile_put8(uint16_t (*tile)[kTP], int row, int f8, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    tile[row][f8 + 2 * u] = static_cast<uint16_t>(w[u] & 0xFFFFu);
    tile[row][f8 + 2 * u + 1] = static_cast<uint16_t>(w[u] >> 16);
  }
}

// 8 elements tile[r8 .. r8+7][col] packed into 16 bytes.
__device__ __forceinline__ uint4 tile_get8_column(const uint16_t (*tile)[kTP], int r8, int col) {
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    w[u] = static_cast<uint32_t>(tile[r8 + 2 * u][col]) | (static_cast<uint32_t>(tile[r8 + 2 * u + 1][col]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// dst[r][kofs[e] + i] = src[row(offsets[e] + i)][r] for the kept rows i of
// expert e, 0 in the padding; row(s) = src_rows[s] or s.
__global__ __launch_bounds__(256) void transpose_groups_kernel(
    const bf16_t* __restrict__ src, const int32_t* __restrict__ src_rows, int R,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kofs, int E, int S, int cap,
    bf16_t* __restrict__ dst, int ldk) {
  __shared__ uint16_t tile[kTile][kTP];  // [slot i][feature]
  __shared__ int e_s, beg_s, n_s;
  const int c0 = blockIdx.x * kTile;  // first padded column of the tile
  const int r0 = blockIdx.y * kTile;
  if (threadIdx.x == 0) {
    int e = -1;
    for (int x = 0; x < E; ++x)
      if (kofs[x] <= c0 && c0 < kofs[x + 1]) e = x;
    e_s = e;
    if (e >= 0) {
      int beg, end;
      expert_rows(offsets, e, S, cap, &beg, &end);
      beg_s = beg + (c0 - kofs[e]);  // grouped row of the tile's first column
      n_s = end - beg_s;             // kept rows from there on
    }
  }
  __syncthreads();
  if (e_s < 0) return;  // past the last expert's range
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int q = threadIdx.x + 256 * h2;
    const int i = q / 8, f8 = (q % 8) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < n_s && r0 + f8 < R) {
      const int sl = beg_s + i;
      const int row = src_rows != nullptr ? src_rows[sl] : sl;
      v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * R + r0 + f8);
    }
    tile_put8(tile, i, f8, v);
  }
  __syncthreads();
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int q = threadIdx.x + 256 * h2;
    const int r = q / 8, c8 = (q % 8) * 8;
    if (r0 + r < R)
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(r0 + r) * ldk + c0 + c8) = tile_get8_column(tile, c8, r);
  }
}

// One block per routing slot (t, j) with grouped row s: dO[s] = g dy[t]
// (bfloat16, for the dW2 GEMM), rgate[s] = g, and dyb = dy[t] . b2[e], the
// bias part of the gate gradient (its other part, a[s] . (dy W2), comes from
// the dZ GEMM), summed by a fixed-order tree. A dropped slot gets dyb = 0.
// T: the layer's element type (bfloat16 or float32) of dy, b2 and dO.
template <typename T>
__global__ __launch_bounds__(256) void dout_kernel(const T* __restrict__ dy, const int32_t* __restrict__ token_slot,
                                                   const int32_t* __restrict__ topk_idx,
                                                   const float* __restrict__ gate, const T* __restrict__ b2, int d,
                                                   int K, T* __restrict__ dO, float* __restrict__ rgate,
                                                   float* __restrict__ dyb) {
  __shared__ float red[256];
  const int tj = blockIdx.x;
  const int t = tj / K;
  const int s = token_slot[tj];
  if (s < 0) {
    if (threadIdx.x == 0) dyb[tj] = 0.0f;
    return;
  }
  const float g = gate[tj];
  if (threadIdx.x == 0) rgate[s] = g;
  const T* dyr = dy + static_cast<size_t>(t) * d;
  const T* br = b2 != nullptr ? b2 + static_cast<size_t>(topk_idx[tj]) * d : nullptr;
  T* dor = dO + static_cast<size_t>(s) * d;
  float acc = 0.0f;
  for (int n = threadIdx.x; n < d; n += 256) {
    const float v = Elem<T>::load(dyr + n);
    Elem<T>::store(dor + n, g * v);
    if (br != nullptr) acc = fmaf(v, Elem<T>::load(br + n), acc);
  }
  if (b2 == nullptr) {
    if (threadIdx.x == 0) dyb[tj] = 0.0f;
    return;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) dyb[tj] = red[0];
}

// One thread per grouped row: the dZ GEMM's 64-column partial sums of a . u,
// as eight interleaved running sums (block c goes to sum c mod 8, eight loads
// in flight) added pairwise at the end: a fixed order.
__global__ __launch_bounds__(64) void dgate_sum_kernel(const float* __restrict__ dgp, int ncb, int S,
                                                       float* __restrict__ dgs) {
  const int s = blockIdx.x * 64 + threadIdx.x;
  if (s >= S) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int c = 0;
  for (; c + 8 <= ncb; c += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += dgp[static_cast<size_t>(c + u) * S + s];
  }
  for (int u = 0; c < ncb; ++c, ++u) acc[u] += dgp[static_cast<size_t>(c) * S + s];
  dgs[s] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// One wave per token, lane = expert: d loss / d gate logits.
__global__ __launch_bounds__(256) void router_backward_kernel(
    const float* __restrict__ logits, const float* __restrict__ br, int bias_select,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ gate, const float* __restrict__ dgs,
    const float* __restrict__ dyb, const int32_t* __restrict__ token_slot, const int32_t* __restrict__ counts,
    int T, int E, int K, int gate_mode, float daux, float dz, float* __restrict__ dl) {
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (t >= T) return;
  auto dgate = [&](int j) {  // d loss / d g of slot (t, j): 0 for a dropped slot
    const int s = token_slot[t * K + j];
    return s >= 0 ? dgs[s] + dyb[t * K + j] : 0.0f;
  };
  const bool on = lane < E;
  float gl = -INFINITY;
  if (on) {
    gl = logits[static_cast<size_t>(t) * E + lane];
    if (bias_select && br != nullptr) gl -= br[lane];
  }
  float m = gl;
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float ex = on ? expf(gl - m) : 0.0f;
  float sum = ex;
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float p = ex / sum;
  float dlv = 0.0f, dp = 0.0f;
  if (gate_mode == 0) {  // renormalised: dl[c_j] = g_j (dg_j - sum_i g_i dg_i)
    float sdot = 0.0f;
    for (int j = 0; j < K; ++j) sdot += gate[t * K + j] * dgate(j);
    for (int j = 0; j < K; ++j)
      if (topk_idx[t * K + j] == lane) dlv += gate[t * K + j] * (dgate(j) - sdot);
  } else {  // raw: g_j = p[c_j]
    for (int j = 0; j < K; ++j)
      if (topk_idx[t * K + j] == lane) dp += dgate(j);
  }
  if (on && daux != 0.0f) {
    const float f = static_cast<float>(counts[lane]) / (static_cast<float>(T) * static_cast<float>(K));
    dp += daux * static_cast<float>(E) * f / static_cast<float>(T);
  }
  float pdp = on ? p * dp : 0.0f;
  for (int off = 32; off > 0; off >>= 1) pdp += __shfl_xor(pdp, off);
  // z-loss: d (lse_t^2 / T) / d l = 2 lse_t p / T
  const float dzl = dz != 0.0f ? dz * (2.0f / static_cast<float>(T)) * (m + logf(sum)) * p : 0.0f;
  if (on) dl[static_cast<size_t>(t) * E + lane] = dlv + p * (dp - pdp) + dzl;
}

// dh[t] = sum_j dX[slot(t, j)] (ascending j, kept slots) + sum_e dl[t][e] W_r[k][e].
// Block: 16 tokens; a thread keeps one row of W_r in registers across them.
// EP = E padded to 8, 16, 32 or 64 (padding entries are 0). A thread covers KV
// consecutive features (16-byte loads of dX when KV = 4) and keeps their W_r
// rows in registers across the block's tokens.
constexpr int kDhTokens = 16;
template <int EP, int KV, typename Tout>
__global__ __launch_bounds__(256) void dh_kernel(const float* __restrict__ dX, const int32_t* __restrict__ token_slot,
                                                 const float* __restrict__ dl, const float* __restrict__ Wr, int T,
                                                 int d, int E, int K, Tout* __restrict__ dh) {
  __shared__ float dl_s[kDhTokens][EP];
  __shared__ int slot_s[kDhTokens][8];
  const int t0 = blockIdx.x * kDhTokens;
  for (int i = threadIdx.x; i < kDhTokens * EP; i += 256) {
    const int tt = t0 + i / EP, e = i % EP;
    dl_s[i / EP][e] = (tt < T && e < E) ? dl[static_cast<size_t>(tt) * E + e] : 0.0f;
  }
  for (int i = threadIdx.x; i < kDhTokens * 8; i += 256) {
    const int tt = t0 + i / 8, j = i % 8;
    slot_s[i / 8][j] = (tt < T && j < K) ? token_slot[tt * K + j] : -1;
  }
  __syncthreads();
  for (int k0 = threadIdx.x * KV; k0 < d; k0 += 256 * KV) {  // d is a multiple of 8
    float wr[KV][EP];
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int e = 0; e < EP; ++e) wr[v][e] = e < E ? Wr[static_cast<size_t>(k0 + v) * E + e] : 0.0f;
    for (int i = 0; i < kDhTokens; ++i) {
      const int t = t0 + i;
      if (t >= T) break;
      float acc[KV];
#pragma unroll
      for (int v = 0; v < KV; ++v) acc[v] = 0.0f;
      for (int j = 0; j < K; ++j) {
        const int s = slot_s[i][j];
        if (s < 0) continue;
        const float* src = dX + static_cast<size_t>(s) * d + k0;
        if constexpr (KV == 4) {
          const float4 x = *reinterpret_cast<const float4*>(src);
          acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
        } else {
#pragma unroll
          for (int v = 0; v < KV; ++v) acc[v] += src[v];
        }
      }
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        float r = 0.0f;
#pragma unroll
        for (int e = 0; e < EP; ++e) r = fmaf(dl_s[i][e], wr[v][e], r);
        Elem<Tout>::store(dh + static_cast<size_t>(t) * d + k0 + v, acc[v] + r);
      }
    }
  }
}

// Partial sums over chunks of kWrChunk tokens: part[c][k][e] = sum_t h[t][k] dl[t][e];
// column e of chunk c, row k: one thread, tokens in order.
constexpr int kWrChunk = 256;
template <int EP, typename Tin>
__global__ __launch_bounds__(256) void dwr_partial_kernel(const Tin* __restrict__ h, const float* __restrict__ dl,
                                                          int T, int d, int E, float* __restrict__ part) {
  __shared__ float dl_s[kWrChunk][EP + 1];
  const int c = blockIdx.y;
  const int t0 = c * kWrChunk;
  const int nt = min(kWrChunk, T - t0);
  for (int i = threadIdx.x; i < kWrChunk * EP; i += 256) {
    const int tt = i / EP, e = i % EP;
    dl_s[tt][e] = (tt < nt && e < E) ? dl[static_cast<size_t>(t0 + tt) * E + e] : 0.0f;
  }
  __syncthreads();
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d) return;
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0f;
  for (int tt = 0; tt < nt; ++tt) {
    const float hv = Elem<Tin>::load(h + static_cast<size_t>(t0 + tt) * d + k);
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = fmaf(hv, dl_s[tt][e], acc[e]);  // padding columns are 0
  }
  float* dst = part + (static_cast<size_t>(c) * d + k) * E;
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (e < E) dst[e] = acc[e];
}

// dW_r[k][e] = sum over chunks in order; db_r[e] = sum_t dl[t][e] in order.
__global__ __launch_bounds__(256) void dwr_final_kernel(const float* __restrict__ part, int nchunk,
                                                        const float* __restrict__ dl, int T, int d, int E,
                                                        float* __restrict__ dWr, float* __restrict__ dbr) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t n = static_cast<size_t>(d) * E;
  if (i < n) {
    float s = 0.0f;
    for (int c = 0; c < nchunk; ++c) s += part[static_cast<size_t>(c) * n + i];
    dWr[i] = s;
  }
  if (dbr != nullptr && blockIdx.x == 0 && threadIdx.x < E) {
    float s = 0.0f;
    for (int t = 0; t < T; ++t) s += dl[static_cast<size_t>(t) * E + threadIdx.x];
    dbr[threadIdx.x] = s;
  }
}

// out[e][c] = sum over the kept grouped rows of expert e of src[row][c] (in order).
template <typename T>
__global__ __launch_bounds__(256) void group_colsum_kernel(const T* __restrict__ src, int C,
                                                           const int32_t* __restrict__ offsets, int S, int cap,
                                                           float* __restrict__ out) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  int beg, end;
  expert_rows(offsets, e, S, cap, &beg, &end);
  float s = 0.0f;
  for (int r = beg; r < end; ++r) s += Elem<T>::load(src + static_cast<size_t>(r) * C + c);
  out[static_cast<size_t>(e) * C + c] = s;
}

// Float32 layers, one block per grouped row s: from u = dy W2 of the row
// (the second GEMM's input gradient before the gate), dA = g u,
// dgs[s] = sum_j a[s][j] u[s][j] (the gate gradient's term from the expert
// output; a fixed-order tree), and dZ = dA * act'(z): SwiGLU [dz1 | dz3] with
// dz1 = dA z3 SiLU'(z1), dz3 = dA SiLU(z1); GELU dz = dA GELU'(z). Rows of
// dropped slots hold values that nothing reads.
__global__ __launch_bounds__(256) void dz_f32_kernel(const float* __restrict__ u, const float* __restrict__ z,
                                                     const float* __restrict__ a, const float* __restrict__ rgate,
                                                     int w, int act, float* __restrict__ dZ,
                                                     float* __restrict__ dgs) {
  __shared__ float red[256];
  const int s = blockIdx.x;
  const float g = rgate[s];
  const float* ur = u + static_cast<size_t>(s) * w;
  const float* ar = a + static_cast<size_t>(s) * w;
  const int zw = act == 1 ? 2 * w : w;
  const float* zr = z + static_cast<size_t>(s) * zw;
  float* dzr = dZ + static_cast<size_t>(s) * zw;
  float acc = 0.0f;
  for (int j = threadIdx.x; j < w; j += 256) {
    const float uv = ur[j];
    acc = fmaf(ar[j], uv, acc);
    const float da = g * uv;
    if (act == 1) {
      const float z1 = zr[j], z3 = zr[w + j];
      const float sg = 1.0f / (1.0f + expf(-z1));
      dzr[j] = da * z3 * (sg * (1.0f + z1 * (1.0f - sg)));
      dzr[w + j] = da * (z1 * sg);
    } else {
      const float x = zr[j];
      dzr[j] = da * (0.5f * (1.0f + erff(x * 0.70710678118654752440f)) +
                     x * expf(-0.5f * x * x) * 0.39894228040143267794f);
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgs[s] = red[0];
}

unsigned grid1d(size_t n) {
  const size_t b = (n + 255) / 256;
  return static_cast<unsigned>(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int S, int cap, int32_t* kofs, hipStream_t st) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, st, offsets, E, S, cap, kofs);
  return hipGetLastError();
}

hipError_t launch_transpose_groups(const void* src, const int32_t* src_rows, int R, const int32_t* offsets,
                                   const int32_t* kofs, int E, int S, int cap, void* dst, int ldk,
                                   hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ldk / kTile), static_cast<unsigned>((R + kTile - 1) / kTile));
  hipLaunchKernelGGL(transpose_groups_kernel, grid, dim3(256), 0, st, static_cast<const bf16_t*>(src), src_rows,
                     R, offsets, kofs, E, S, cap, static_cast<bf16_t*>(dst), ldk);
  return hipGetLastError();
}

hipError_t launch_dout(const void* dy, const int32_t* token_slot, const int32_t* topk_idx, const float* gate,
                       const void* b2, int T, int d, int K, void* dO, float* rgate, float* dyb, bool bf16,
                       hipStream_t st) {
  if (bf16) {
    hipLaunchKernelGGL(dout_kernel<bf16_t>, dim3(static_cast<unsigned>(T * K)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(dy), token_slot, topk_idx, gate, static_cast<const bf16_t*>(b2), d,
                       K, static_cast<bf16_t*>(dO), rgate, dyb);
  } else {
    hipLaunchKernelGGL(dout_kernel<float>, dim3(static_cast<unsigned>(T * K)), dim3(256), 0, st,
                       static_cast<const float*>(dy), token_slot, topk_idx, gate, static_cast<const float*>(b2), d, K,
                       static_cast<float*>(dO), rgate, dyb);
  }
  return hipGetLastError();
}

hipError_t launch_dgate_sum(const float* dgp, int ncb, int S, float* dgs, hipStream_t st) {
  hipLaunchKernelGGL(dgate_sum_kernel, dim3(static_cast<unsigned>((S + 63) / 64)), dim3(64), 0, st, dgp, ncb, S,
                     dgs);
  return hipGetLastError();
}

hipError_t launch_router_backward(const float* logits, const float* br, int bias_select, const int32_t* topk_idx,
                                  const float* gate, const float* dgs, const float* dyb,
                                  const int32_t* token_slot, const int32_t* counts, int T, int E, int K,
                                  int gate_mode, float daux, float dz, float* dl, hipStream_t st) {
  hipLaunchKernelGGL(router_backward_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, st, logits,
                     br, bias_select, topk_idx, gate, dgs, dyb, token_slot, counts, T, E, K, gate_mode, daux, dz,
                     dl);
  return hipGetLastError();
}

template <int EP, typename Tout>
hipError_t launch_dh_ep(const float* dX, const int32_t* token_slot, const float* dl, const float* Wr, int T, int d,
                        int E, int K, void* dh, hipStream_t st) {
  constexpr int KV = EP <= 16 ? 4 : 1;
  hipLaunchKernelGGL((dh_kernel<EP, KV, Tout>), dim3(static_cast<unsigned>((T + kDhTokens - 1) / kDhTokens)),
                     dim3(256), 0, st, dX, token_slot, dl, Wr, T, d, E, K, static_cast<Tout*>(dh));
  return hipGetLastError();
}

template <typename Tout>
hipError_t launch_dh_t(const float* dX, const int32_t* token_slot, const float* dl, const float* Wr, int T, int d,
                       int E, int K, void* dh, hipStream_t st) {
  if (E <= 8) return launch_dh_ep<8, Tout>(dX, token_slot, dl, Wr, T, d, E, K, dh, st);
  if (E <= 16) return launch_dh_ep<16, Tout>(dX, token_slot, dl, Wr, T, d, E, K, dh, st);
  if (E <= 32) return launch_dh_ep<32, Tout>(dX, token_slot, dl, Wr, T, d, E, K, dh, st);
  return launch_dh_ep<64, Tout>(dX, token_slot, dl, Wr, T, d, E, K, dh, st);
}

hipError_t launch_dh(const float* dX, const int32_t* token_slot, const float* dl, const float* Wr, int T, int d,
                     int E, int K, void* dh, bool bf16, hipStream_t st) {
  return bf16 ? launch_dh_t<bf16_t>(dX, token_slot, dl, Wr, T, d, E, K, dh, st)
              : launch_dh_t<float>(dX, token_slot, dl, Wr, T, d, E, K, dh, st);
}

int dwr_chunks(int T) { return (T + kWrChunk - 1) / kWrChunk; }

template <typename Tin>
void launch_dwr_partial(const Tin* hb, const float* dl, int T, int d, int E, float* part, dim3 grid,
                        hipStream_t st) {
  if (E <= 8) hipLaunchKernelGGL((dwr_partial_kernel<8, Tin>), grid, dim3(256), 0, st, hb, dl, T, d, E, part);
  else if (E <= 16) hipLaunchKernelGGL((dwr_partial_kernel<16, Tin>), grid, dim3(256), 0, st, hb, dl, T, d, E, part);
  else if (E <= 32) hipLaunchKernelGGL((dwr_partial_kernel<32, Tin>), grid, dim3(256), 0, st, hb, dl, T, d, E, part);
  else hipLaunchKernelGGL((dwr_partial_kernel<64, Tin>), grid, dim3(256), 0, st, hb, dl, T, d, E, part);
}

hipError_t launch_dwr(const void* h, const float* dl, int T, int d, int E, float* part, float* dWr, float* dbr,
                      bool bf16, hipStream_t st) {
  const int nc = dwr_chunks(T);
  const dim3 grid(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(nc));
  if (bf16) launch_dwr_partial(static_cast<const bf16_t*>(h), dl, T, d, E, part, grid, st);
  else launch_dwr_partial(static_cast<const float*>(h), dl, T, d, E, part, grid, st);
  hipLaunchKernelGGL(dwr_final_kernel, dim3(static_cast<unsigned>((static_cast<size_t>(d) * E + 255) / 256)),
                     dim3(256), 0, st, part, nc, dl, T, d, E, dWr, dbr);
  return hipGetLastError();
}

hipError_t launch_group_colsum(const void* src, int C, const int32_t* offsets, int E, int S, int cap, float* out,
                               bool bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((C + 255) / 256), static_cast<unsigned>(E));
  if (bf16) {
    hipLaunchKernelGGL(group_colsum_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(src), C,
                       offsets, S, cap, out);
  } else {
    hipLaunchKernelGGL(group_colsum_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(src), C,
                       offsets, S, cap, out);
  }
  return hipGetLastError();
}

hipError_t launch_dz_f32(const float* u, const float* z, const float* a, const float* rgate, int S, int width,
                         int act, float* dZ, float* dgs, hipStream_t st) {
  hipLaunchKernelGGL(dz_f32_kernel, dim3(static_cast<unsigned>(S)), dim3(256), 0, st, u, z, a, rgate, width, act, dZ,
                     dgs);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = 0u;
}
}  // namespace

// Zero `bytes` bytes (a multiple of 4) with a kernel, so that the call can be
// captured in a graph.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (p == nullptr || bytes == 0) return hipSuccess;
  const size_t n = bytes / 4;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid1d(n)), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace moe

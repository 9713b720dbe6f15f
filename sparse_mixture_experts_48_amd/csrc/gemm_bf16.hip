// Expert FFN GEMMs in bfloat16 on gfx950 MFMA, fp32 accumulation.
//
// Each expert is a full feed-forward block (Lensa ML explainer "Mixture of
// Experts", Step 1) that runs only on the rows routed to it (maptheai.com
// "Mixture of Experts", section "The mechanism"). After grouping, expert e
// owns rows offsets[e] .. offsets[e+1]-1 of h_perm, so the layer is a grouped
// GEMM over ragged row counts (Step 5: any number of tokens per expert).
//
//   GEMM1 SwiGLU: a = SiLU(x W1) * (x W3)      x: [rows][d], W1/W3 stored [E][w][d]
//   GEMM1 GELU:   a = GELU(x W1 + b1)
//   GEMM2:        o = a W2 (+ b2)               W2 stored [E][d][w]
//                 -> o_perm (float32), or, for K = 1, y[token] = gate * o
//
// Both operands keep the reduction dimension contiguous, so every lane loads
// 16-byte runs along k for either operand. The sum over k does not care which
// k a lane's MFMA slot stands for, as long as the A and B fragments use the
// same assignment; the loaders below exploit that to read long contiguous runs.
//
// Two kernel families; the host picks one from T (an upper bound on the rows
// of any expert):
//  * gemm_tile_kernel: BM x BN tiles on v_mfma_f32_32x32x16_bf16, LDS double
//    buffer, tiles enumerated over (expert m-tiles) x (n-tiles) on the device
//    from expert_offsets, so no host synchronisation is needed.
//  * gemm_stream_kernel (rows per expert <= 32): every wave streams NR x 16
//    weight rows over the whole reduction with v_mfma_f32_16x16x32_bf16, the
//    weights as the M operand and up to 32 token rows as N; weights are read
//    from HBM exactly once, which is what bounds decode-sized batches.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

enum { G1_SWIGLU = 0, G1_GELU = 1, G2_OPERM = 2, G2_FUSED_Y = 3 };

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct GemmParams {
  const bf16_t* x;          // [S][Kd] grouped input rows (or h, through x_rows)
  const int32_t* x_rows;    // nullable: grouped row s is row x_rows[s] of x
  const int32_t* offsets;   // [E+1]
  const bf16_t* B;          // [E][N][Kd]
  const bf16_t* B3;         // [E][N][Kd] (SwiGLU) or null
  const bf16_t* bias;       // [E][N] or null
  void* out;                // a: bf16 [S][N]; o_perm: f32 [S][N]; fused: y bf16 [T][N]
  const int32_t* slot_token;
  const float* gate;        // topk_gate [T] (K = 1)
  int E, N, Kd;
  int n_mt;                 // m-tile slots in the grid (upper bound)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ float epilogue_g1(int mode, float v1, float v3, const bf16_t* bias, int e,
                                             int N, int col) {
  if (mode == G1_SWIGLU) return silu(v1) * v3;
  float z = v1;
  if (bias != nullptr) z += bf16_to_f32(bias[static_cast<size_t>(e) * N + col]);
  return gelu_exact(z);
}

// ---------------------------------------------------------------------------- tiled kernel
//
// Block: 256 threads = 2 x 2 waves; tile = BM grouped rows x BN weight rows;
// k staged 64 at a time in a double-buffered LDS tile that is filled by
// direct global-to-LDS loads (global_load_lds_dwordx4): no staging
// registers, no LDS store instructions. One stage per iteration:
//   barrier (this stage's loads have landed in every wave)
//   -> read all of this stage's MFMA fragments into registers
//   -> issue the loads of the next stage into the other buffer
//   -> 64 MFMAs per wave.
// Nothing reads LDS between issuing a stage's loads and the next barrier.
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r sits at
// c ^ ((r & 7) ^ ((r >> 3) & 1)), so the 16-byte fragment reads of 8 or 16
// consecutive rows fall in distinct bank groups. A direct load fills 64
// consecutive chunk slots (8 rows) per wave instruction; each lane fetches
// the global chunk that belongs in its slot. Chunks past the end of the
// reduction come from a 16-byte zero constant.
//
// The weights are the MFMA M operand and the tokens the N operand, so lane l
// of a 32x32 accumulator holds token l % 32 and four consecutive output
// columns per register group; the epilogue stores 4 values at once.
//
// SwiGLU: the BN weight rows of a block are, per wave, WTN/2 rows of W1
// followed by the same WTN/2 rows of W3, so the two products that meet in
// SiLU(x W1) * (x W3) sit in the same lane and register.

constexpr int kBK = 64;   // k per stage: 8 chunks of 8 bf16

__device__ const u32x4_t kZeroChunk = {0u, 0u, 0u, 0u};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 8 + (chunk ^ ((row & 7) ^ ((row >> 3) & 1)));
}

__device__ __forceinline__ void lds_dma16(const void* gsrc, u32x4_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(gsrc),
                                   (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmParams p) {
  constexpr int WM = 2, WN = 2;
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_IN = BM / 32;        // direct-load instructions per wave per stage (8 rows each)
  constexpr int B_IN = BN / 32;
  constexpr int NCOLS = BN / NMAT;     // output columns per block
  static_assert(TM >= 1 && TN >= NMAT && A_IN >= 1 && B_IN >= 1, "tile too small");

  // One array per buffer, so that reads of one buffer are known not to alias
  // the direct loads that fill the other.
  __shared__ u32x4_t A0[BM * 8], B0[BN * 8], A1[BM * 8], B1[BN * 8];

  const int mt = blockIdx.x % p.n_mt;
  const int nt = blockIdx.x / p.n_mt;
  int e, row0, rows;
  if (!find_m_tile(p.offsets, p.E, BM, mt, &e, &row0, &rows)) return;
  const int n0 = nt * NCOLS;

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wid = tid / 64;
  const int wm = wid / WN, wn = wid % WN;
  const int Kd = p.Kd, N = p.N;

  // weight row j of the block tile -> (matrix, output column)
  auto brow_col = [&](int j, int* mat) {
    if constexpr (NMAT == 2) {
      const int g = j / WTN, w = j % WTN;
      *mat = w >= WTN / 2;
      return n0 + g * (WTN / 2) + (w % (WTN / 2));
    } else {
      *mat = 0;
      return n0 + j;
    }
  };

  // Direct-load sources. Wave wid, instruction u fills slots
  // [(wid*A_IN + u)*64, +64): rows (wid*A_IN + u)*8 + lane/8, physical chunk
  // lane%8, i.e. logical chunk (lane%8) ^ f(row).
  // 32-bit element offsets (every operand matrix has fewer than 2^31 elements).
  // The logical chunk of instruction u depends only on the parity of u.
  const int kc_even = ((lane % 8) ^ ((lane / 8) & 7)) * 8;
  const int kc_odd = ((lane % 8) ^ ((lane / 8) & 7) ^ 1) * 8;
  int a_off[A_IN];
#pragma unroll
  for (int u = 0; u < A_IN; ++u) {
    const int r = (wid * A_IN + u) * 8 + lane / 8;
    const int s = row0 + min(r, rows - 1);
    const int src_row = (p.x_rows != nullptr) ? p.x_rows[s] : s;
    a_off[u] = src_row * Kd + (((wid * A_IN + u) & 1) ? kc_odd : kc_even);
  }
  const bf16_t* Bexp = p.B + static_cast<size_t>(e) * N * Kd;
  const bf16_t* B3exp = (NMAT == 2) ? p.B3 + static_cast<size_t>(e) * N * Kd : Bexp;
  int b_off[B_IN];
#pragma unroll
  for (int u = 0; u < B_IN; ++u) {
    const int j = (wid * B_IN + u) * 8 + lane / 8;
    int mat;
    const int n = min(brow_col(j, &mat), N - 1);
    // SwiGLU: a wave's B instructions alternate between W1 and W3 row blocks
    b_off[u] = n * Kd + (((wid * B_IN + u) & 1) ? kc_odd : kc_even);
    (void)mat;
  }
  auto issue_stage = [&](int k0, u32x4_t* As, u32x4_t* Bs) {
#pragma unroll
    for (int u = 0; u < A_IN; ++u) {
      const int kc = ((wid * A_IN + u) & 1) ? kc_odd : kc_even;
      const void* g = (k0 + kc < Kd) ? static_cast<const void*>(p.x + a_off[u] + k0)
                                     : static_cast<const void*>(&kZeroChunk);
      lds_dma16(g, As + (wid * A_IN + u) * 64);
    }
#pragma unroll
    for (int u = 0; u < B_IN; ++u) {
      const int j0 = (wid * B_IN + u) * 8;
      int mat;
      (void)brow_col(j0, &mat);  // all 8 rows of one instruction come from the same matrix
      const int kc = ((wid * B_IN + u) & 1) ? kc_odd : kc_even;
      const bf16_t* base = (NMAT == 2 && mat) ? B3exp : Bexp;
      const void* g = (k0 + kc < Kd) ? static_cast<const void*>(base + b_off[u] + k0)
                                     : static_cast<const void*>(&kZeroChunk);
      lds_dma16(g, Bs + (wid * B_IN + u) * 64);
    }
  };

  f32x16_t acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  const int frow = lane % 32;
  const int fsub = lane / 32;  // which of the two 8-wide k chunks of a 16-k step
  const int nk = (Kd + kBK - 1) / kBK;

  // One stage: barrier (stage kt landed everywhere), first fragments, loads of
  // stage kt+1 into the other buffer pair, then MFMAs of k-step ks while the
  // fragments of ks+1 are read.
  auto run_stage = [&](int kt, const u32x4_t* As, const u32x4_t* Bs, u32x4_t* An, u32x4_t* Bn) {
    __syncthreads();
    bf16x8_t wf[kBK / 16][TN], xf[kBK / 16][TM];
    auto read = [&](int ks) {
      const int c = ks * 2 + fsub;
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[ks][j] = as_bf16x8(Bs[swz(wn * WTN + j * 32 + frow, c)]);
#pragma unroll
      for (int i = 0; i < TM; ++i) xf[ks][i] = as_bf16x8(As[swz(wm * WTM + i * 32 + frow, c)]);
    };
    read(0);
    if (kt + 1 < nk) issue_stage((kt + 1) * kBK, An, Bn);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      if (ks + 1 < kBK / 16) read(ks + 1);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][j], xf[ks][i], acc[j][i], 0, 0, 0);
    }
  };

  issue_stage(0, A0, B0);
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {  // straight-line pair of stages: no merge point for acc
    run_stage(kt, A0, B0, A1, B1);
    run_stage(kt + 1, A1, B1, A0, B0);
  }
  if (kt < nk) run_stage(kt, A0, B0, A1, B1);

  // Epilogue. Accumulator (j, i), register r: token = i*32 + lane%32 of the
  // wave's rows; weight row = j*32 + (r/4)*8 + (lane/32)*4 + r%4.
  constexpr int TNO = TN / NMAT;  // output column tiles per wave
#pragma unroll
  for (int j = 0; j < TNO; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = wm * WTM + i * 32 + (lane % 32);
      if (rl >= rows) continue;
      const int s = row0 + rl;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (WTN / NMAT) + j * 32 + g * 8 + (lane / 32) * 4;
        if (n >= N) continue;  // N % 8 == 0: four columns are all in or all out
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v1 = acc[j][i][g * 4 + q];
          if (MODE == G1_SWIGLU || MODE == G1_GELU) {
            v[q] = epilogue_g1(MODE, v1, acc[NMAT == 2 ? j + TNO : j][i][g * 4 + q], p.bias, e, N, n + q);
          } else {
            v[q] = v1;
            if (p.bias != nullptr) v[q] += bf16_to_f32(p.bias[static_cast<size_t>(e) * N + n + q]);
          }
        }
        if (MODE == G1_SWIGLU || MODE == G1_GELU) {
          *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else if (MODE == G2_OPERM) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + static_cast<size_t>(s) * N + n) =
              f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          const int t = p.slot_token[s];
          const float gt = p.gate[t];
          *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(t) * N + n) =
              u32x2_t{pack_bf16x2(gt * v[0], gt * v[1]), pack_bf16x2(gt * v[2], gt * v[3])};
        }
      }
    }
}

// ---------------------------------------------------------------------------- streaming kernel

constexpr int kStreamWaves = 4;
constexpr int kKS = 128;  // k per step: 4 loads of 32 contiguous k (8 per lane group) per row

template <int MODE, int NR, int MC>
__global__ __launch_bounds__(kStreamWaves * 64) void gemm_stream_kernel(GemmParams p, int n_groups) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  const int e = blockIdx.x / n_groups;
  const int grp = blockIdx.x % n_groups;
  const int beg = p.offsets[e];
  const int rows = p.offsets[e + 1] - beg;
  if (rows <= 0) return;
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int n_base = (grp * kStreamWaves + wave) * NR * 16;
  const int N = p.N, Kd = p.Kd;
  if (n_base >= N) return;
  const int lr = lane % 16;     // row inside a 16-row fragment
  const int lg = lane / 16;     // lane group: 8 k values inside each 32-wide run

  const bf16_t* wsrc[NMAT][NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int n = min(n_base + q * 16 + lr, N - 1);
    wsrc[0][q] = p.B + (static_cast<size_t>(e) * N + n) * Kd + lg * 8;
    if (NMAT == 2) wsrc[NMAT - 1][q] = p.B3 + (static_cast<size_t>(e) * N + n) * Kd + lg * 8;
  }
  const bf16_t* xsrc[MC];
  bool xok[MC];
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const int r = c * 16 + lr;
    xok[c] = r < rows;
    const int s = beg + min(r, rows - 1);
    xsrc[c] = p.x + static_cast<size_t>(p.x_rows != nullptr ? p.x_rows[s] : s) * Kd + lg * 8;
  }

  f32x4_t acc[NMAT][NR][MC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
      for (int c = 0; c < MC; ++c) acc[m][q][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wreg[2][NMAT][NR][4];
  u32x4_t xreg[2][MC][4];
  auto load = [&](int slot, int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool kin = k0 + u * 32 + lg * 8 < Kd;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int q = 0; q < NR; ++q)
          wreg[slot][m][q][u] = kin ? *reinterpret_cast<const u32x4_t*>(wsrc[m][q] + k0 + u * 32)
                                    : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < MC; ++c)
        xreg[slot][c][u] = (kin && xok[c]) ? *reinterpret_cast<const u32x4_t*>(xsrc[c] + k0 + u * 32)
                                           : u32x4_t{0, 0, 0, 0};
    }
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
          for (int c = 0; c < MC; ++c)
            acc[m][q][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(wreg[slot][m][q][u]), as_bf16x8(xreg[slot][c][u]), acc[m][q][c], 0, 0, 0);
  };

  const int nk = (Kd + kKS - 1) / kKS;
  load(0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    load(1, (kt + 1) * kKS);
    compute(0);
    if (kt + 2 < nk) load(0, (kt + 2) * kKS);
    compute(1);
  }
  if (kt < nk) compute(0);

  // 16x16 accumulator layout: lane l holds column l%16 (a token row) and
  // rows (l/16)*4 + r (four consecutive output columns n).
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int n = n_base + q * 16 + lg * 4;
    if (n >= N) continue;  // N is a multiple of 8: a group of four is all in or all out
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int r = c * 16 + lr;
      if (r >= rows) continue;
      const int s = beg + r;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (MODE == G1_SWIGLU || MODE == G1_GELU) {
          v[i] = epilogue_g1(MODE, acc[0][q][c][i], acc[NMAT - 1][q][c][i], p.bias, e, N, n + i);
        } else {
          v[i] = acc[0][q][c][i];
          if (p.bias != nullptr) v[i] += bf16_to_f32(p.bias[static_cast<size_t>(e) * N + n + i]);
        }
      }
      if (MODE == G1_SWIGLU || MODE == G1_GELU) {
        *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else if (MODE == G2_OPERM) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + static_cast<size_t>(s) * N + n) =
            f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
        const int t = p.slot_token[s];
        const float g = p.gate[t];
        *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(t) * N + n) =
            u32x2_t{pack_bf16x2(g * v[0], g * v[1]), pack_bf16x2(g * v[2], g * v[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------- launch

template <int BM, int BN, int MODE>
hipError_t launch_tile(GemmParams p, int S, hipStream_t st) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  p.n_mt = (S + BM - 1) / BM + min(p.E, S);
  const int n_nt = (p.N + BN / NMAT - 1) / (BN / NMAT);
  const size_t grid = static_cast<size_t>(p.n_mt) * n_nt;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, MODE>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Large tiles when the grid still covers the chip a few times over.
template <int MODE>
hipError_t launch_tile_auto(GemmParams p, int S, hipStream_t st) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  const long big = static_cast<long>((S + 255) / 256 + min(p.E, S)) * ((p.N + 256 / NMAT - 1) / (256 / NMAT));
  if (big >= 4 * 256) return launch_tile<256, 256, MODE>(p, S, st);
  const long mid = static_cast<long>((S + 255) / 256 + min(p.E, S)) * ((p.N + 128 / NMAT - 1) / (128 / NMAT));
  if (mid >= 2 * 256) return launch_tile<256, 128, MODE>(p, S, st);
  return launch_tile<128, 128, MODE>(p, S, st);
}

template <int MODE, int NR>
hipError_t launch_stream(GemmParams p, int max_rows, hipStream_t st) {
  const int n_groups = (p.N + kStreamWaves * NR * 16 - 1) / (kStreamWaves * NR * 16);
  const dim3 grid(static_cast<unsigned>(p.E * n_groups));
  if (max_rows <= 16) {
    hipLaunchKernelGGL((gemm_stream_kernel<MODE, NR, 1>), grid, dim3(kStreamWaves * 64), 0, st, p, n_groups);
  } else {
    hipLaunchKernelGGL((gemm_stream_kernel<MODE, NR, 2>), grid, dim3(kStreamWaves * 64), 0, st, p, n_groups);
  }
  return hipGetLastError();
}

constexpr int kStreamMaxRows = 32;

}  // namespace

hipError_t launch_gemm1_bf16(const FfnArgs& f, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(f.x);
  p.x_rows = f.x_rows;
  p.offsets = f.offsets;
  p.B = static_cast<const bf16_t*>(f.W1);
  p.B3 = static_cast<const bf16_t*>(f.W3);
  p.bias = static_cast<const bf16_t*>(f.b1);
  p.out = f.a;
  p.E = f.E;
  p.N = f.width;
  p.Kd = f.d;
  const bool swiglu = f.act == 1;
  if (f.max_rows_per_expert <= kStreamMaxRows) {
    return swiglu ? launch_stream<G1_SWIGLU, 2>(p, f.max_rows_per_expert, st)
                  : launch_stream<G1_GELU, 2>(p, f.max_rows_per_expert, st);
  }
  return swiglu ? launch_tile_auto<G1_SWIGLU>(p, f.S, st) : launch_tile_auto<G1_GELU>(p, f.S, st);
}

hipError_t launch_gemm2_bf16(const FfnArgs& f, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(f.a);
  p.offsets = f.offsets;
  p.B = static_cast<const bf16_t*>(f.W2);
  p.B3 = nullptr;
  p.bias = static_cast<const bf16_t*>(f.b2);
  p.E = f.E;
  p.N = f.d;
  p.Kd = f.width;
  if (f.fused_y) {
    p.out = f.y;
    p.slot_token = f.slot_token;
    p.gate = f.topk_gate;
  } else {
    p.out = f.o_perm;
  }
  if (f.max_rows_per_expert <= kStreamMaxRows) {
    return f.fused_y ? launch_stream<G2_FUSED_Y, 1>(p, f.max_rows_per_expert, st)
                     : launch_stream<G2_OPERM, 1>(p, f.max_rows_per_expert, st);
  }
  return f.fused_y ? launch_tile_auto<G2_FUSED_Y>(p, f.S, st) : launch_tile_auto<G2_OPERM>(p, f.S, st);
}

}  // namespace moe

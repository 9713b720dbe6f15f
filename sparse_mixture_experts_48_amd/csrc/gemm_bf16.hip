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
  const bf16_t* x;          // [S][Kd] grouped input rows
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

constexpr int kBK = 64;          // k per LDS stage
constexpr int kLDA = kBK + 8;    // padded row (bf16): 144 bytes, conflict-free 16-byte reads

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int CPR = kBK / 8;                 // 16-byte chunks per row per stage
  constexpr int A_CH = BM * CPR / NT;          // A chunks per thread
  constexpr int B_CH = BN * CPR / NT;          // B chunks per thread per matrix
  static_assert(A_CH * NT == BM * CPR && B_CH * NT == BN * CPR, "tile/threads mismatch");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");

  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t* A_s = smem;                               // [2][BM][kLDA]
  bf16_t* B_s = smem + 2 * BM * kLDA;               // [2][NMAT][BN][kLDA]

  const int mt = blockIdx.x % p.n_mt;
  const int nt = blockIdx.x / p.n_mt;
  int e, row0, rows;
  if (!find_m_tile(p.offsets, p.E, BM, mt, &e, &row0, &rows)) return;
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wid = tid / 64;
  const int wm = wid / WN, wn = wid % WN;
  const int Kd = p.Kd, N = p.N;

  // global source pointers for this thread's chunks (rows clamped in range)
  const bf16_t* a_src[A_CH];
  int a_kc[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT;
    const int r = min(c / CPR, rows - 1);
    a_kc[i] = (c % CPR) * 8;
    a_src[i] = p.x + static_cast<size_t>(row0 + r) * Kd + a_kc[i];
  }
  const bf16_t* b_src[NMAT][B_CH];
  int b_kc[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT;
    const int n = min(n0 + c / CPR, N - 1);
    b_kc[i] = (c % CPR) * 8;
    b_src[0][i] = p.B + (static_cast<size_t>(e) * N + n) * Kd + b_kc[i];
    if (NMAT == 2) b_src[NMAT - 1][i] = p.B3 + (static_cast<size_t>(e) * N + n) * Kd + b_kc[i];
  }

  u32x4_t a_reg[A_CH];
  u32x4_t b_reg[NMAT][B_CH];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      a_reg[i] = (k0 + a_kc[i] < Kd) ? *reinterpret_cast<const u32x4_t*>(a_src[i] + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        b_reg[m][i] = (k0 + b_kc[i] < Kd) ? *reinterpret_cast<const u32x4_t*>(b_src[m][i] + k0)
                                          : u32x4_t{0, 0, 0, 0};
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(A_s + (buf * BM + c / CPR) * kLDA + (c % CPR) * 8) = a_reg[i];
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NT;
        *reinterpret_cast<u32x4_t*>(B_s + ((buf * NMAT + m) * BN + c / CPR) * kLDA + (c % CPR) * 8) =
            b_reg[m][i];
      }
  };

  f32x16_t acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;

  const int nk = (Kd + kBK - 1) / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int frow = lane % 32;
  const int fk = (lane / 32) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[TM];
      bf16x8_t bfr[NMAT][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
            A_s + (buf * BM + wm * WTM + i * 32 + frow) * kLDA + kk * 16 + fk));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[m][j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
              B_s + ((buf * NMAT + m) * BN + wn * WTN + j * 32 + frow) * kLDA + kk * 16 + fk));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j], acc[m][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue. 32x32 accumulator layout: lane l holds column l%32 and rows
  // (r/4)*8 + (l/32)*4 + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + (lane % 32);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * WTM + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
        if (rl >= rows) continue;
        const int s = row0 + rl;
        if (MODE == G1_SWIGLU || MODE == G1_GELU) {
          const float v = epilogue_g1(MODE, acc[0][i][j][r], acc[NMAT - 1][i][j][r], p.bias, e, N, col);
          static_cast<bf16_t*>(p.out)[static_cast<size_t>(s) * N + col] = f32_to_bf16(v);
        } else {
          float v = acc[0][i][j][r];
          if (p.bias != nullptr) v += bf16_to_f32(p.bias[static_cast<size_t>(e) * N + col]);
          if (MODE == G2_OPERM) {
            static_cast<float*>(p.out)[static_cast<size_t>(s) * N + col] = v;
          } else {
            const int t = p.slot_token[s];
            static_cast<bf16_t*>(p.out)[static_cast<size_t>(t) * N + col] = f32_to_bf16(p.gate[t] * v);
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------- streaming kernel

constexpr int kStreamWaves = 4;
constexpr int kKS = 128;  // k per step: 4 lane groups x 32 contiguous values

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
  const int lg = lane / 16;     // lane group: which 32-wide k run

  const bf16_t* wsrc[NMAT][NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int n = min(n_base + q * 16 + lr, N - 1);
    wsrc[0][q] = p.B + (static_cast<size_t>(e) * N + n) * Kd + lg * 32;
    if (NMAT == 2) wsrc[NMAT - 1][q] = p.B3 + (static_cast<size_t>(e) * N + n) * Kd + lg * 32;
  }
  const bf16_t* xsrc[MC];
  bool xok[MC];
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const int r = c * 16 + lr;
    xok[c] = r < rows;
    xsrc[c] = p.x + static_cast<size_t>(beg + min(r, rows - 1)) * Kd + lg * 32;
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
      const bool kin = k0 + lg * 32 + u * 8 < Kd;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int q = 0; q < NR; ++q)
          wreg[slot][m][q][u] = kin ? *reinterpret_cast<const u32x4_t*>(wsrc[m][q] + k0 + u * 8)
                                    : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < MC; ++c)
        xreg[slot][c][u] = (kin && xok[c]) ? *reinterpret_cast<const u32x4_t*>(xsrc[c] + k0 + u * 8)
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

template <int BM, int BN, int WM, int WN, int MODE>
hipError_t launch_tile(GemmParams p, int S, hipStream_t st) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  const size_t smem = static_cast<size_t>(2) * (BM + NMAT * BN) * kLDA * sizeof(bf16_t);
  static bool attr_set = false;  // per template instance
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, WM, WN, MODE>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  p.n_mt = (S + BM - 1) / BM + min(p.E, S);
  const int n_nt = (p.N + BN - 1) / BN;
  const size_t grid = static_cast<size_t>(p.n_mt) * n_nt;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, WN, MODE>), dim3(static_cast<unsigned>(grid)),
                     dim3(WM * WN * 64), smem, st, p);
  return hipGetLastError();
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
  return swiglu ? launch_tile<128, 128, 2, 2, G1_SWIGLU>(p, f.S, st)
                : launch_tile<128, 128, 2, 2, G1_GELU>(p, f.S, st);
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
  return f.fused_y ? launch_tile<128, 128, 2, 2, G2_FUSED_Y>(p, f.S, st)
                   : launch_tile<128, 128, 2, 2, G2_OPERM>(p, f.S, st);
}

}  // namespace moe

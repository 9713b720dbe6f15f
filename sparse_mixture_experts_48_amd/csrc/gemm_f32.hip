// Expert FFN GEMMs in float32 (layers stored in float32, such as the micro
// model of the Curionode plate "Mixture of Experts.", section "Workshop").
//
// Same grouped structure as the bfloat16 kernels (each expert runs on its own
// contiguous rows; tiles enumerated on the device from expert_offsets), with
// 64 x 64 tiles of plain fp32 fused multiply-adds: 256 threads, 4 x 4 outputs
// per thread, k staged through LDS 16 at a time.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

enum { F_G1_SWIGLU = 0, F_G1_GELU = 1, F_G2_OPERM = 2, F_G2_FUSED_Y = 3 };

constexpr int kFBM = 64, kFBN = 64, kFBK = 16, kFPad = 4;

struct F32Params {
  const float* x;          // [S][Kd] grouped rows (or h, through x_rows)
  const int32_t* x_rows;   // nullable: grouped row s is row x_rows[s] of x
  const int32_t* offsets;  // [E+1]
  const float* B;          // [E][N][Kd]
  const float* B3;         // [E][N][Kd] or null
  const float* bias;       // [E][N] or null
  void* out;
  const int32_t* slot_token;
  const float* gate;
  int E, N, Kd, S, n_mt;
  int cap;                 // rows each expert processes at most
};

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int NMAT = (MODE == F_G1_SWIGLU) ? 2 : 1;
  __shared__ __align__(16) float A_s[kFBK][kFBM + kFPad];
  __shared__ __align__(16) float B_s[NMAT][kFBK][kFBN + kFPad];

  const int mt = blockIdx.x % p.n_mt;
  const int nt = blockIdx.x / p.n_mt;
  int e, row0, rows;
  const WaveTiles wt = wave_tiles(p.offsets, p.E, p.S, p.cap, kFBM);
  if (mt >= wt.total) return;
  wave_tile_owner(wt, kFBM, mt, &e, &row0, &rows);
  const int n0 = nt * kFBN;
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int N = p.N, Kd = p.Kd;

  // loader: thread -> (row = tid / 4, k = (tid % 4) * 4), four consecutive k
  const int lrow = tid / 4, lk = (tid % 4) * 4;
  const int arow = row0 + min(lrow, rows - 1);
  const float* a_src = p.x + static_cast<size_t>(p.x_rows != nullptr ? p.x_rows[arow] : arow) * Kd + lk;
  const int bn = min(n0 + lrow, N - 1);
  const float* b_src[NMAT];
  b_src[0] = p.B + (static_cast<size_t>(e) * N + bn) * Kd + lk;
  if (NMAT == 2) b_src[NMAT - 1] = p.B3 + (static_cast<size_t>(e) * N + bn) * Kd + lk;

  float acc[NMAT][4][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.0f;

  for (int k0 = 0; k0 < Kd; k0 += kFBK) {
    const bool kin = k0 + lk < Kd;  // Kd is a multiple of 8, lk a multiple of 4
    const float4 av = kin ? *reinterpret_cast<const float4*>(a_src + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
    A_s[lk + 0][lrow] = av.x;
    A_s[lk + 1][lrow] = av.y;
    A_s[lk + 2][lrow] = av.z;
    A_s[lk + 3][lrow] = av.w;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const float4 bv = kin ? *reinterpret_cast<const float4*>(b_src[m] + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
      B_s[m][lk + 0][lrow] = bv.x;
      B_s[m][lk + 1][lrow] = bv.y;
      B_s[m][lk + 2][lrow] = bv.z;
      B_s[m][lk + 3][lrow] = bv.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFBK; ++k) {
      const float4 a4 = *reinterpret_cast<const float4*>(&A_s[k][ty * 4]);
      const float av4[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const float4 b4 = *reinterpret_cast<const float4*>(&B_s[m][k][tx * 4]);
        const float bv4[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(av4[i], bv4[j], acc[m][i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = ty * 4 + i;
    if (rl >= rows) continue;
    const int s = row0 + rl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      if (MODE == F_G1_SWIGLU) {
        static_cast<float*>(p.out)[static_cast<size_t>(s) * N + col] = silu(acc[0][i][j]) * acc[NMAT - 1][i][j];
      } else if (MODE == F_G1_GELU) {
        float z = acc[0][i][j];
        if (p.bias != nullptr) z += p.bias[static_cast<size_t>(e) * N + col];
        static_cast<float*>(p.out)[static_cast<size_t>(s) * N + col] = gelu_exact(z);
      } else {
        float v = acc[0][i][j];
        if (p.bias != nullptr) v += p.bias[static_cast<size_t>(e) * N + col];
        if (MODE == F_G2_OPERM) {
          static_cast<float*>(p.out)[static_cast<size_t>(s) * N + col] = v;
        } else {
          const int t = p.slot_token[s];
          static_cast<float*>(p.out)[static_cast<size_t>(t) * N + col] = p.gate[t] * v;
        }
      }
    }
  }
}

template <int MODE>
hipError_t launch_f32(F32Params p, int S, hipStream_t st) {
  p.n_mt = (S + kFBM - 1) / kFBM + min(p.E, S);
  const int n_nt = (p.N + kFBN - 1) / kFBN;
  hipLaunchKernelGGL((gemm_f32_kernel<MODE>), dim3(static_cast<unsigned>(static_cast<size_t>(p.n_mt) * n_nt)),
                     dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_f32(const FfnArgs& f, hipStream_t st) {
  F32Params p{};
  p.x = static_cast<const float*>(f.x);
  p.x_rows = f.x_rows;
  p.offsets = f.offsets;
  p.B = static_cast<const float*>(f.W1);
  p.B3 = static_cast<const float*>(f.W3);
  p.bias = static_cast<const float*>(f.b1);
  p.out = f.a;
  p.E = f.E;
  p.N = f.width;
  p.Kd = f.d;
  p.S = f.S;
  p.cap = f.cap;
  return f.act == 1 ? launch_f32<F_G1_SWIGLU>(p, f.S, st) : launch_f32<F_G1_GELU>(p, f.S, st);
}

hipError_t launch_gemm2_f32(const FfnArgs& f, hipStream_t st) {
  F32Params p{};
  p.x = static_cast<const float*>(f.a);
  p.offsets = f.offsets;
  p.B = static_cast<const float*>(f.W2);
  p.bias = static_cast<const float*>(f.b2);
  p.E = f.E;
  p.N = f.d;
  p.Kd = f.width;
  p.S = f.S;
  p.cap = f.cap;
  if (f.fused_y) {
    p.out = f.y;
    p.slot_token = f.slot_token;
    p.gate = f.topk_gate;
    return launch_f32<F_G2_FUSED_Y>(p, f.S, st);
  }
  p.out = f.o_perm;
  return launch_f32<F_G2_OPERM>(p, f.S, st);
}

}  // namespace moe

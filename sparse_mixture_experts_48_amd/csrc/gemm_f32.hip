// Expert FFN GEMMs in float32 (layers stored in float32, such as the micro
// model of the Curionode plate "Mixture of Experts.", section "Workshop"), and
// the float32 GEMMs of the layer's backward pass.
//
// Same grouped structure as the bfloat16 kernels (each expert runs on its own
// contiguous rows; tiles enumerated on the device from expert_offsets), on
// float32 MFMA (v_mfma_f32_32x32x2_f32). These layers are small and bound by
// latency, so the operands go straight from memory (L2) into registers, with
// a ring of loads in flight and no LDS stage or barrier: a wave computes a
// 32 x 32 block of outputs, a block of four waves 64 x 64.
//
// MFMA layout: the weights are the A operand (32 output columns n), the
// grouped rows the B operand (32 rows s), so lane l of an accumulator holds
// row l % 32 and, in register r, column (r / 4) * 8 + (l / 32) * 4 + r % 4:
// four consecutive columns per register group. Each k-block of 8 is four
// MFMAs; in MFMA i, lanes 0..31 hold k = 8j + i and lanes 32..63 hold
// k = 8j + 4 + i, so a lane loads the four consecutive k of its half with one
// 16-byte load when k is contiguous in memory. Both operands use the same
// assignment, so the sum is the same whatever k a slot stands for.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef float f32x16v __attribute__((ext_vector_type(16)));

enum {
  F_G1_SWIGLU = 0, F_G1_GELU = 1, F_G2_OPERM = 2, F_G2_FUSED_Y = 3,
  F_Z = 4,      // backward: pre-activations z (SwiGLU: [x W1 | x W3] in rows of 2N) and a = act(z)
  F_PLAIN = 5   // out[s][n] = the sum, float32
};

constexpr int kFT = 64;     // rows and columns of a block tile
constexpr int kFRing = 4;   // k-blocks of 8 in flight per wave

struct F32Params {
  const float* x;          // grouped rows [.][lda] (or rows of x through x_rows)
  const int32_t* x_rows;   // nullable: grouped row s is row x_rows[s] of x
  int lda;                 // row stride of x (floats)
  int x_nrows;             // rows of x
  const int32_t* offsets;  // [E+1]
  const float* B;          // per expert: BT ? [Kd][N] : [N][Kd]
  const float* B3;         // second matrix (SwiGLU: W3; backward dX: W3 for the second k-segment) or null
  const float* bias;       // [E][N] or null
  void* out;
  void* out_act;           // F_Z: a = act(z) [S][N]
  const int32_t* slot_token;
  const float* gate;
  int E, N, Kd, S, n_mt, ldo;
  int cap;                 // rows each expert processes at most
  int act;                 // F_Z: 1 SwiGLU, 0 GELU
  int x_koff2;             // backward dX with B3: column offset in x of the second k-segment
};

__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// One 8-k block of operands of a lane: four consecutive k of row `row` of a
// row-major matrix with k contiguous (16 bytes), or of a matrix stored with k
// as the row index (four strided loads, coalesced across the lanes).
template <bool KT>
__device__ __forceinline__ float4 load_k4(const float* base, int row, int k, int ld) {
  if constexpr (KT) {
    return make_float4(base[static_cast<size_t>(k) * ld + row], base[static_cast<size_t>(k + 1) * ld + row],
                       base[static_cast<size_t>(k + 2) * ld + row], base[static_cast<size_t>(k + 3) * ld + row]);
  } else {
    return *reinterpret_cast<const float4*>(base + static_cast<size_t>(row) * ld + k);
  }
}

// Sum over k in [0, Kd) of A(n, k) x(s, k) for the wave's 32 x 32 block into
// acc[m] for each of NMAT weight matrices.
template <int NMAT, bool BT>
__device__ __forceinline__ void f32_mma(f32x16v* acc, const float* const* Bm, int bn, int ldb, const float* xrow,
                                        int Kd) {
  const int lane = threadIdx.x % 64;
  const int kh = (lane / 32) * 4;
  const int nkb = Kd / 8;  // Kd is a multiple of 8
  float4 wr[kFRing][NMAT], xr[kFRing];
  auto load = [&](int slot, int kb) {
    const int k = min(kb, nkb - 1) * 8 + kh;  // past the end: reload the last block (never used)
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wr[slot][m] = load_k4<BT>(Bm[m], bn, k, ldb);
    xr[slot] = *reinterpret_cast<const float4*>(xrow + k);
  };
#pragma unroll
  for (int i = 0; i < kFRing - 1; ++i) load(i, i);
  for (int kb0 = 0; kb0 < nkb; kb0 += kFRing) {
#pragma unroll
    for (int r = 0; r < kFRing; ++r) {
      if (kb0 + r < nkb) {
        load((r + kFRing - 1) % kFRing, kb0 + r + kFRing - 1);
        const float xs[4] = {xr[r].x, xr[r].y, xr[r].z, xr[r].w};
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const float ws[4] = {wr[r][m].x, wr[r][m].y, wr[r][m].z, wr[r][m].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(ws[i], xs[i], acc[m], 0, 0, 0);
        }
      }
    }
  }
}

template <int MODE, bool BT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int NMAT = (MODE == F_G1_SWIGLU || (MODE == F_Z)) ? 2 : 1;  // F_Z GELU uses acc[0] only
  const int mt = blockIdx.x % p.n_mt;
  const int nt = blockIdx.x / p.n_mt;
  const WaveTiles wt = wave_tiles(p.offsets, p.E, p.S, p.cap, kFT);
  if (mt >= wt.total) return;
  int e, row0, rows;
  wave_tile_owner(wt, kFT, mt, &e, &row0, &rows);
  const int lane = threadIdx.x % 64, wid = threadIdx.x / 64;
  const int wr0 = (wid / 2) * 32;  // the wave's first row of the tile
  const int wn0 = (wid % 2) * 32;  // ... and first column
  if (wr0 >= rows) return;         // no rows for this wave
  const int N = p.N, Kd = p.Kd;
  const int n0 = nt * kFT + wn0;
  if (n0 >= N) return;
  const bool swiglu_z = MODE == F_Z && p.act == 1;

  // operand rows of this lane (clamped: extra rows and columns are computed, never stored)
  const int bn = min(n0 + lane % 32, N - 1);
  const int rl = wr0 + lane % 32;
  const int s = row0 + min(rl, rows - 1);
  const int xr_row = p.x_rows != nullptr ? p.x_rows[s] : s;
  const float* xrow = p.x + static_cast<size_t>(xr_row) * p.lda;
  const size_t eoff = static_cast<size_t>(e) * N * Kd;
  const int ldb = BT ? N : Kd;

  f32x16v acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
  if constexpr (MODE == F_Z) {
    const float* Bm[2] = {p.B + eoff, swiglu_z ? p.B3 + eoff : p.B + eoff};
    if (swiglu_z) f32_mma<2, BT>(acc, Bm, bn, ldb, xrow, Kd);
    else f32_mma<1, BT>(acc, Bm, bn, ldb, xrow, Kd);
  } else if constexpr (MODE == F_PLAIN) {
    const float* Bm[1] = {p.B + eoff};
    f32_mma<1, BT>(acc, Bm, bn, ldb, xrow, Kd);
    if (p.B3 != nullptr) {  // a second k-segment: x columns from x_koff2 against B3
      const float* Bm3[1] = {p.B3 + eoff};
      f32_mma<1, BT>(acc, Bm3, bn, ldb, xrow + p.x_koff2, Kd);
    }
  } else {
    const float* Bm[NMAT];
    Bm[0] = p.B + eoff;
    if constexpr (NMAT == 2) Bm[1] = p.B3 + eoff;
    f32_mma<NMAT, BT>(acc, Bm, bn, ldb, xrow, Kd);
  }

  if (rl >= rows) return;
  const int srow = row0 + rl;
  // Inputs of the epilogue loaded before its first store (a load placed after a
  // store waits for it): the bias of the four column groups (columns past N
  // clamped) and, for the K = 1 scatter, the row's token and gate.
  const bool has_bias = (MODE == F_G1_GELU || MODE == F_Z || MODE == F_G2_OPERM || MODE == F_G2_FUSED_Y) &&
                        p.bias != nullptr && !swiglu_z;
  float4 bias4[4];
  if (has_bias) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bias4[g] = *reinterpret_cast<const float4*>(p.bias + static_cast<size_t>(e) * N +
                                                  min(n0 + g * 8 + (lane / 32) * 4, N - 4));
  }
  int fy_t = 0;
  float fy_g = 0.0f;
  if constexpr (MODE == F_G2_FUSED_Y) {
    fy_t = p.slot_token[srow];
    fy_g = p.gate[fy_t];
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = n0 + g * 8 + (lane / 32) * 4;
    if (n >= N) continue;  // N is a multiple of 8: four columns are all in or all out
    const float bq[4] = {has_bias ? bias4[g].x : 0.0f, has_bias ? bias4[g].y : 0.0f, has_bias ? bias4[g].z : 0.0f,
                         has_bias ? bias4[g].w : 0.0f};
    float v[4], v3[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = acc[0][g * 4 + q];
      v3[q] = acc[1][g * 4 + q];
    }
    if constexpr (MODE == F_G1_SWIGLU) {
      store4(static_cast<float*>(p.out) + static_cast<size_t>(srow) * N + n, silu(v[0]) * v3[0], silu(v[1]) * v3[1],
             silu(v[2]) * v3[2], silu(v[3]) * v3[3]);
    } else if constexpr (MODE == F_G1_GELU) {
      float z[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) z[q] = gelu_exact(has_bias ? v[q] + bq[q] : v[q]);
      store4(static_cast<float*>(p.out) + static_cast<size_t>(srow) * N + n, z[0], z[1], z[2], z[3]);
    } else if constexpr (MODE == F_Z) {
      float* zrow = static_cast<float*>(p.out) + static_cast<size_t>(srow) * (swiglu_z ? 2 * N : N);
      float* arow = static_cast<float*>(p.out_act) + static_cast<size_t>(srow) * N;
      if (swiglu_z) {
        store4(zrow + n, v[0], v[1], v[2], v[3]);
        store4(zrow + N + n, v3[0], v3[1], v3[2], v3[3]);
        store4(arow + n, silu(v[0]) * v3[0], silu(v[1]) * v3[1], silu(v[2]) * v3[2], silu(v[3]) * v3[3]);
      } else {
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) z[q] = has_bias ? v[q] + bq[q] : v[q];
        store4(zrow + n, z[0], z[1], z[2], z[3]);
        store4(arow + n, gelu_exact(z[0]), gelu_exact(z[1]), gelu_exact(z[2]), gelu_exact(z[3]));
      }
    } else if constexpr (MODE == F_PLAIN) {
      store4(static_cast<float*>(p.out) + static_cast<size_t>(srow) * p.ldo + n, v[0], v[1], v[2], v[3]);
    } else {
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = has_bias ? v[q] + bq[q] : v[q];
      if constexpr (MODE == F_G2_OPERM) {
        store4(static_cast<float*>(p.out) + static_cast<size_t>(srow) * N + n, o[0], o[1], o[2], o[3]);
      } else {
        store4(static_cast<float*>(p.out) + static_cast<size_t>(fy_t) * N + n, fy_g * o[0], fy_g * o[1],
               fy_g * o[2], fy_g * o[3]);
      }
    }
  }
}

template <int MODE, bool BT>
hipError_t launch_f32(F32Params p, int S, hipStream_t st) {
  p.n_mt = (S + kFT - 1) / kFT + min(p.E, S);
  const int n_nt = (p.N + kFT - 1) / kFT;
  hipLaunchKernelGGL((gemm_f32_kernel<MODE, BT>), dim3(static_cast<unsigned>(static_cast<size_t>(p.n_mt) * n_nt)),
                     dim3(256), 0, st, p);
  return hipGetLastError();
}

// Weight gradients: for every expert e, C_e[m][n] = sum over its kept grouped
// rows s of A[s][m] B[row(s)][n] (A [S][M], B rows through b_rows), rows m < split
// to out [E][split][N], the rest to out2 [E][M - split][N]. The reduction runs
// over the slots in order of 8-slot blocks (rows past the expert's end count 0).
struct F32WgradParams {
  const float* A;          // [S][M]
  const float* Bx;         // [.][N]
  const int32_t* b_rows;   // nullable: row s of B is b_rows[s]
  const int32_t* offsets;
  float* out;
  float* out2;
  int E, M, N, S, cap, split;
};

__global__ __launch_bounds__(256) void wgrad_f32_kernel(F32WgradParams p) {
  const int e = blockIdx.z;
  const int lane = threadIdx.x % 64, wid = threadIdx.x / 64;
  const int m0 = blockIdx.y * kFT + (wid / 2) * 32;  // the MFMA's A side: output rows m
  const int n0 = blockIdx.x * kFT + (wid % 2) * 32;  // B side: output columns n
  if (m0 >= p.M || n0 >= p.N) return;
  int beg, end;
  expert_rows(p.offsets, e, p.S, p.cap, &beg, &end);
  const int mm = min(m0 + lane % 32, p.M - 1);
  const int nn = min(n0 + lane % 32, p.N - 1);
  const int kh = (lane / 32) * 4;
  f32x16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int k0 = beg; k0 < end; k0 += 8) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = k0 + kh + i;
      const bool in = s < end;
      const int sc = min(s, end - 1);
      const int br = p.b_rows != nullptr ? p.b_rows[sc] : sc;
      const float a = p.A[static_cast<size_t>(sc) * p.M + mm];
      const float b = p.Bx[static_cast<size_t>(br) * p.N + nn];
      av[i] = in ? a : 0.0f;
      bv[i] = in ? b : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[i], acc, 0, 0, 0);
  }
  // lane l: column n0 + l % 32; register r: row m0 + (r / 4) * 8 + (l / 32) * 4 + r % 4
  const int n = n0 + lane % 32;
  if (n >= p.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + (r / 4) * 8 + (lane / 32) * 4 + r % 4;
    if (m >= p.M) continue;
    float* dst = m < p.split ? p.out + (static_cast<size_t>(e) * p.split + m) * p.N + n
                             : p.out2 + (static_cast<size_t>(e) * (p.M - p.split) + (m - p.split)) * p.N + n;
    *dst = acc[r];
  }
}

}  // namespace

hipError_t launch_gemm1_f32(const FfnArgs& f, hipStream_t st) {
  F32Params p{};
  p.x = static_cast<const float*>(f.x);
  p.x_rows = f.x_rows;
  p.lda = f.d;
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
  return f.act == 1 ? launch_f32<F_G1_SWIGLU, false>(p, f.S, st) : launch_f32<F_G1_GELU, false>(p, f.S, st);
}

hipError_t launch_gemm2_f32(const FfnArgs& f, hipStream_t st) {
  F32Params p{};
  p.x = static_cast<const float*>(f.a);
  p.lda = f.width;
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
    return launch_f32<F_G2_FUSED_Y, false>(p, f.S, st);
  }
  p.out = f.o_perm;
  return launch_f32<F_G2_OPERM, false>(p, f.S, st);
}

// Backward: z and a = act(z) of the grouped rows (x rows through x_rows).
hipError_t launch_bwd_z_f32(const FfnArgs& f, void* z, void* a, hipStream_t st) {
  F32Params p{};
  p.x = static_cast<const float*>(f.x);
  p.x_rows = f.x_rows;
  p.lda = f.d;
  p.offsets = f.offsets;
  p.B = static_cast<const float*>(f.W1);
  p.B3 = static_cast<const float*>(f.W3);
  p.bias = static_cast<const float*>(f.b1);
  p.out = z;
  p.out_act = a;
  p.act = f.act;
  p.E = f.E;
  p.N = f.width;
  p.Kd = f.d;
  p.S = f.S;
  p.cap = f.cap;
  return launch_f32<F_Z, false>(p, f.S, st);
}

// Backward: out[s][n] = sum_k x[row(s)][k] B_e[k][n] (B stored with k as the
// row index: [E][Kd][N]), plus, with B3, sum_k x[row(s)][koff2 + k] B3_e[k][n].
hipError_t launch_bwd_grouped_f32(const float* x, const int32_t* x_rows, int lda, int S, const int32_t* offsets,
                                  int cap, int E, const float* B, const float* B3, int koff2, int N, int Kd,
                                  float* out, hipStream_t st) {
  F32Params p{};
  p.x = x;
  p.x_rows = x_rows;
  p.lda = lda;
  p.offsets = offsets;
  p.B = B;
  p.B3 = B3;
  p.x_koff2 = koff2;
  p.out = out;
  p.ldo = N;
  p.E = E;
  p.N = N;
  p.Kd = Kd;
  p.S = S;
  p.cap = cap;
  return launch_f32<F_PLAIN, true>(p, S, st);
}

hipError_t launch_bwd_wgrad_f32(const float* A, int M, const float* Bx, const int32_t* b_rows, int N,
                                const int32_t* offsets, int S, int cap, int E, float* out, float* out2, int split,
                                hipStream_t st) {
  F32WgradParams p{A, Bx, b_rows, offsets, out, out2, E, M, N, S, cap, split};
  const dim3 grid(static_cast<unsigned>((N + kFT - 1) / kFT), static_cast<unsigned>((M + kFT - 1) / kFT),
                  static_cast<unsigned>(E));
  hipLaunchKernelGGL(wgrad_f32_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe

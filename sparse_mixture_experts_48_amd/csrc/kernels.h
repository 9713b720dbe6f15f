// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Token tiling of the router; the grouping kernels reuse it so that the
// router's per-block histograms line up with the grouping blocks.
struct RouteTiling {
  int EP;   // experts padded to 8, 16, 32 or 64
  int NW;   // waves per block of the narrow layout; 0 selects the wide or broadcast layout
  int TB;   // tokens per block (at most 32)
  int NB;   // blocks
};
RouteTiling route_tiling(int64_t T, int64_t E);

struct RouteArgs {
  const void* h;
  const float* Wr;
  const float* br;
  int T, d, E, K, gate;
  int32_t* topk_idx;
  float* topk_gate;
  float* logits;      // nullable
  int32_t* blk_hist;  // [NB][E]
  float* blk_psum;    // [NB][E]
  int bias_select = 0;  // 1: br steers the choice only; softmax and gates use h . W_r
  const float* noise = nullptr;  // [T][E] added to the logits after the bias, or null
  float* blk_z = nullptr;        // [NB] per-block sums of lse^2 (z-loss), or null
};

hipError_t launch_route(const RouteArgs& a, const RouteTiling& rt, bool bf16, hipStream_t st);
hipError_t launch_hist(const int32_t* topk_idx, int T, int E, int K, const RouteTiling& rt,
                       int32_t* blk_hist, hipStream_t st);
// z_loss (nullable) = sum of blk_z / T; blk_z may be null when z_loss is.
hipError_t launch_finalize(const int32_t* blk_hist, const float* blk_psum, const float* blk_z, int NB, int T,
                           int E, int K, int32_t* blk_base, int32_t* counts, int32_t* offsets, float* prob_mean,
                           float* aux, float* z_loss, hipStream_t st);
hipError_t launch_zero_outputs(int E, int32_t* counts, int32_t* offsets, float* prob_mean, float* aux,
                               float* z_loss, hipStream_t st);

// The router's per-block partials and what the finalize kernel forms from them
// (outputs nullable), for the fused statistics-and-grouping launch below.
struct FinArgs {
  const int32_t* blk_hist = nullptr;
  const float* blk_psum = nullptr;
  const float* blk_z = nullptr;
  int NB = 0;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  float* prob_mean = nullptr;
  float* aux = nullptr;
  float* z_loss = nullptr;
};

// Stable grouping: slot ranks, token_slot, slot_token and the gathered rows.
// With cap < INT_MAX, a slot whose rank in its expert's group is cap or more is
// dropped: its token_slot entry is -1.
hipError_t launch_permute(const int32_t* topk_idx, const int32_t* blk_base, const int32_t* offsets, int T,
                          int E, int K, int cap, const RouteTiling& rt, const void* h, size_t row_bytes,
                          void* h_perm, int32_t* slot_token, int32_t* token_slot, hipStream_t st);
// Statistics and grouping in one launch: every grouping block forms the
// statistics (bit for bit as launch_finalize; block 0 writes them) and its own
// base rows, then groups.
hipError_t launch_finalize_permute(const FinArgs& fin, const int32_t* topk_idx, int T, int E, int K, int cap,
                                   const RouteTiling& rt, const void* h, size_t row_bytes, void* h_perm,
                                   int32_t* slot_token, int32_t* token_slot, hipStream_t st);

// Expert GEMMs over the grouped rows.
struct FfnArgs {
  int S, d, E, K, width, act;  // S = T*K grouped rows
  bool bf16;
  const void* x;               // grouped rows [S][d], or h [T][d] read through x_rows
  const int32_t* x_rows;       // nullable: GEMM1 reads row x_rows[s] of x for grouped row s
  const int32_t* offsets;      // [E+1]
  const void* W1; const void* b1; const void* W3; const void* W2; const void* b2;
  void* a;                     // hidden activations [S][width], dtype (workspace)
  float* o_perm;               // [S][d] float32; unused when fused_y
  // K = 1 fused gated scatter: y[slot_token[s]] = gate[slot_token[s]] * o[s]
  bool fused_y;
  void* y;
  const int32_t* slot_token;
  const float* topk_gate;
  int max_rows_per_expert;     // host-known bound (min(T, cap)) used to pick the kernel family
  int cap;                     // rows each expert processes at most (INT_MAX: dropless)
  float* tail_part;            // nullable: gemm2_tail_bytes of workspace for split tails (bfloat16)
};
// Workspace the bfloat16 second GEMM uses for split tails (0: none are split).
size_t gemm2_tail_bytes(int S, int E, int d, int width, int max_rows_per_expert, bool fused_y);
hipError_t launch_gemm1(const FfnArgs& f, hipStream_t st);
hipError_t launch_gemm2(const FfnArgs& f, hipStream_t st);

hipError_t launch_combine(const float* o_perm, const int32_t* token_slot, const float* topk_gate,
                          int T, int d, int K, bool bf16, void* y, hipStream_t st);

// ---- backward pass (bfloat16 layers)
// First GEMM without its activation: SwiGLU z = [x W1 | x W3] as rows of 2*width,
// GELU z = x W1 + b1; grouped rows as in launch_gemm1; also a = act(z) [S][width].
hipError_t launch_bwd_z_bf16(const FfnArgs& f, void* z, void* a, hipStream_t st);
// For the grouped rows s (dy rows read through slot_token): u = dy W2, dA = rgate[s] u,
// dZ = dA * act'(z) (z as written by launch_bwd_z_bf16; dZ like z, bfloat16), and
// dgp[c][s] = sum over the 64 columns 64c .. 64c+63 of a[s] u (the gate-gradient
// terms; a [S][N] bfloat16). W2 as stored for the forward pass, [E][Kd = d][N = width]
// (read with k as the row index); dgp [ceil(N/64)][S].
constexpr int kDgpColsHost = 64;
hipError_t launch_bwd_dz_bf16(const void* dy, int T, const int32_t* slot_token, int S, const int32_t* offsets,
                              int cap, int E, const void* W2, int N, int Kd, const void* z, int act,
                              const float* rgate, const void* a, float* dgp, void* dZ, hipStream_t st);
// dX[s] = dZ[s] . [W1_e; W3_e] (float32) for the grouped rows s of every expert e
// (the first cap of each group): W1, W3 as stored for the forward pass,
// [E][Kd1 = width][N = d], read with k as the row index; dZ rows of 2 Kd1
// (SwiGLU, [dz1 | dz3]) or Kd1 (W3 null).
hipError_t launch_bwd_dx_bf16(const void* dZ, int S, const int32_t* offsets, int cap, int E, const void* W1,
                              const void* W3, int N, int Kd1, float* out, float* tail_part, hipStream_t st);
// Workspace the dX GEMM uses for split tails (tail_part of launch_bwd_dx_bf16; 0: none are split).
size_t bwd_dx_tail_bytes(int S, int E, int d, int Kd);
// Weight gradients: C_e[m][n] = sum over expert e's kept grouped slots s of X[s][m] B[s][n]
// (X [S][M] bfloat16, read with the slots as rows). B is either the same kind
// of k-major matrix [S][N] (b_kmajor) or a transposed copy [N][ldk] in which
// expert e's slots sit at columns kofs[e] .. kofs[e+1] (whole 64-k stages, zero
// padded). Rows m < split to out [E][split][N], the rest to out2 [E][M - split][N]
// (float32).
hipError_t launch_bwd_wgrad_bf16(const void* X, int M, const void* B, bool b_kmajor, int N, int ldk,
                                 const int32_t* kofs, const int32_t* offsets, int S, int cap, int E, float* out,
                                 float* out2, int split, hipStream_t st);
// Elementwise, transpose and reduction kernels of the backward pass (csrc/backward.hip).
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int S, int cap, int32_t* kofs, hipStream_t st);
hipError_t launch_transpose_groups(const void* src, const int32_t* src_rows, int R, const int32_t* offsets,
                                   const int32_t* kofs, int E, int S, int cap, void* dst, int ldk,
                                   hipStream_t st);
// Per routing slot: dO[s] = g dy[t] (bfloat16), rgate[s] = g, dyb = dy[t] . b2[e] (0 without b2).
hipError_t launch_dout(const void* dy, const int32_t* token_slot, const int32_t* topk_idx, const float* gate,
                       const void* b2, int T, int d, int K, void* dO, float* rgate, float* dyb, bool bf16,
                       hipStream_t st);
// dgs[s] = sum over c of dgp[c][s], c in order (the gate gradient of grouped row s, bias term aside).
hipError_t launch_dgate_sum(const float* dgp, int ncb, int S, float* dgs, hipStream_t st);
// Gate gradient of slot (t, j): dgs[token_slot] + dyb (0 for a dropped slot).
// Also the z-loss term dz * 2 lse p / T when dz != 0 (lse and p of the gate logits).
hipError_t launch_router_backward(const float* logits, const float* br, int bias_select, const int32_t* topk_idx,
                                  const float* gate, const float* dgs, const float* dyb,
                                  const int32_t* token_slot, const int32_t* counts, int T, int E, int K,
                                  int gate_mode, float daux, float dz, float* dl, hipStream_t st);
hipError_t launch_dh(const float* dX, const int32_t* token_slot, const float* dl, const float* Wr, int T, int d,
                     int E, int K, void* dh, bool bf16, hipStream_t st);
int dwr_chunks(int T);
hipError_t launch_dwr(const void* h, const float* dl, int T, int d, int E, float* part, float* dWr, float* dbr,
                      bool bf16, hipStream_t st);
hipError_t launch_group_colsum(const void* src, int C, const int32_t* offsets, int E, int S, int cap, float* out,
                               bool bf16, hipStream_t st);
// ---- backward pass of float32 layers
// z and a = act(z) of the grouped rows (SwiGLU: z = [x W1 | x W3] in rows of 2 width).
hipError_t launch_bwd_z_f32(const FfnArgs& f, void* z, void* a, hipStream_t st);
// out[s][n] = sum_k x[row(s)][k] B_e[k][n] (B [E][Kd][N]), plus with B3 the same
// over columns koff2 .. koff2 + Kd - 1 of x against B3 (grouped rows, first cap of each expert).
hipError_t launch_bwd_grouped_f32(const float* x, const int32_t* x_rows, int lda, int S, const int32_t* offsets,
                                  int cap, int E, const float* B, const float* B3, int koff2, int N, int Kd,
                                  float* out, hipStream_t st);
// C_e[m][n] = sum over expert e's kept rows s of A[s][m] Bx[row(s)][n], rows m < split to
// out [E][split][N], the others to out2.
hipError_t launch_bwd_wgrad_f32(const float* A, int M, const float* Bx, const int32_t* b_rows, int N,
                                const int32_t* offsets, int S, int cap, int E, float* out, float* out2, int split,
                                hipStream_t st);
// Per grouped row: dA = g u, dgs = sum a u, dZ = dA * act'(z) (float32).
hipError_t launch_dz_f32(const float* u, const float* z, const float* a, const float* rgate, int S, int width,
                         int act, float* dZ, float* dgs, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace moe

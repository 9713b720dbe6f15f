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
//  * gemm_tile_kernel: BM x BN tiles on v_mfma_f32_32x32x16_bf16, LDS rings
//    fed by direct loads, tiles enumerated over (expert m-tiles) x (n-tiles) on the device
//    from expert_offsets, so no host synchronisation is needed.
//  * gemm_stream_kernel (rows per expert <= 32): every wave streams NR x 16
//    weight rows over the whole reduction with v_mfma_f32_16x16x32_bf16, the
//    weights as the M operand and up to 32 token rows as N; weights are read
//    from HBM exactly once, which is what bounds decode-sized batches.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

enum {
  G1_SWIGLU = 0, G1_GELU = 1, G2_OPERM = 2, G2_FUSED_Y = 3,
  // backward pass: the first GEMM's pre-activations (SwiGLU: x W1 and x W3,
  // side by side in rows of 2N; GELU: x W1 + b1), and the weight gradients
  G1_SWIGLU_Z = 4, G1_GELU_Z = 5, G_WGRAD = 6,
  // backward pass: dA = dO W2 with the activation's gradient applied in the
  // epilogue, writing dZ (SwiGLU: [dz1 | dz3] in rows of 2N; GELU: dz)
  G2_DZ_SWIGLU = 7, G2_DZ_GELU = 8
};

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
  int S;                    // grouped rows (bound of every grouped-row index)
  int cap;                  // rows each expert processes at most
  int x_nrows;              // rows of x
  int n_mt;                 // m-tile slots in the grid (upper bound)
  // G_WGRAD: for every expert e, C_e[M][N] = sum over k in [kofs[e], kofs[e+1])
  // of x[m][k] B[n][k] (both row-major with row stride ldk; every expert's
  // range is whole 64-k stages, zero-padded); rows m < split go to out
  // ([E][split][N], float32), the rest to out2 ([E][M - split][N]).
  const int32_t* kofs;
  int M, ldk, split;
  float* out2;
  void* out_act;       // G1_*_Z: also the activation a = act(z), bfloat16 [S][N]
  const bf16_t* zin;   // G2_DZ_*: the pre-activations written by G1_*_Z
  // G2_DZ_*: the reduction gives u = dy W2 for the grouped rows; the epilogue
  // takes dA = rgate[s] u and writes, for every 64 columns c of a row, the
  // sum over them of ain[s][c] u[c] to dgp[c / 64][s] (float32).
  const float* rgate;
  const bf16_t* ain;
  float* dgp;
};
constexpr int kDgpCols = 64;  // columns per partial sum of the dZ GEMM's gate-gradient terms

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
// Block: WM x WN waves; tile = BM grouped rows x BN weight rows. k is staged
// 64 at a time (one 128-byte line of every row) through LDS filled by direct
// global-to-LDS loads (buffer_load_dwordx4 ... lds: no staging registers, no LDS
// store instructions). Each operand has a ring of LDS slots and is loaded one
// stage ahead per slot beyond the first: at 256 x 256 three token slots and
// two weight slots (all 160 KB of LDS: tokens two stages ahead, weights one),
// at 128 x 256 three of each (both two stages ahead), at 128 x 128 three and
// two (so that two blocks share a CU).
// Per stage:
//   wait until this wave's loads of the stage have landed (the loads issued
//   after them may stay in flight), barrier (so have every wave's)
//   -> for each of the four 16-k steps: issue a quarter of the loads of the
//      following stages (the operand loaded fewer stages ahead first), into
//      the slots freed by stage kt-1, read the next step's MFMA fragments,
//      run this step's MFMAs.
// The loads are spread over the MFMAs because a wave issues in order: a load
// that waits for room in the memory pipeline holds up every MFMA behind it.
// A compiler fence after each batch keeps the compiler from sinking the loads
// below later fragment reads (it may, since they target other LDS arrays).
// The loads are buffer loads: the k offset of a stage is a scalar added to a
// per-lane byte offset fixed for the whole reduction, so a load costs no
// vector instructions. In the last stage the lanes whose chunk lies past the
// end of the reduction use an offset past the end of the buffer, which the
// range check turns into zeros. Every stage issues the same number of loads
// (stages past the last reload the last one into slots no stage reads), so
// the wait count is the same at every stage; the kernel drains them before
// its epilogue.
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r sits at
// c ^ ((r & 7) ^ ((r >> 3) & 1)): the fragment reads of 8 or 16 consecutive
// rows fall in distinct bank groups. One direct load fills 64 consecutive
// chunk slots (8 rows) per wave instruction; each lane fetches the global
// chunk that belongs in its slot, so 8 lanes cover one row's 128-byte line.
//
// The weights are the MFMA M operand and the tokens the N operand, so lane l
// of a 32x32 accumulator holds token l % 32 and four consecutive output
// columns per register group; the epilogue stores 4 values at once.
//
// SwiGLU: the BN weight rows of a block are, per wave column, WTN/2 rows of W1
// followed by the same WTN/2 rows of W3, so the two products that meet in
// SiLU(x W1) * (x W3) sit in the same lane and register.

constexpr int kBK = 64;          // k per stage
constexpr int kCH = kBK / 8;     // 16-byte chunks per LDS row
constexpr int kRPI = 64 / kCH;   // rows filled by one direct-load wave instruction
constexpr int kTileGroupN = 4;   // n-tiles per group in the XCD-aware block order

__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kCH + (chunk ^ swz_key(row)); }

// Buffer resource over `bytes` bytes at `base` (raw dword buffer; loads at
// byte offsets >= bytes return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane at byte offset voff + soff of the buffer into LDS: the
// wave writes 64 x 16 consecutive bytes at lds_wave_base.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff,
                                           u32x4_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16,
                                           static_cast<int>(voff), soff, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  constexpr bool G1 = (MODE == G1_SWIGLU || MODE == G1_GELU || MODE == G1_SWIGLU_Z || MODE == G1_GELU_Z);
  constexpr bool WGRAD = (MODE == G_WGRAD);
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_IN = BM / (NW * kRPI);  // token-row loads per wave per stage
  constexpr int B_IN = BN / (NW * kRPI);  // weight-row loads per wave per stage
  constexpr int NKS = kBK / 16;           // MFMA k-steps per stage
  constexpr int PER = (A_IN + B_IN + NKS - 1) / NKS;  // loads issued per k-step
  constexpr int NCOLS = BN / NMAT;        // output columns per block
  static_assert(TM >= 1 && TN >= NMAT && A_IN >= 1 && B_IN >= 1, "tile too small");
  static_assert(WTM % 32 == 0 && WTN % (32 * NMAT) == 0, "wave tile");
  // LDS rings: NAS token slots and NBS weight slots; an operand with n slots is
  // loaded n - 1 stages ahead. Tokens get three slots and weights two (one stage
  // ahead) when that lets two blocks share a CU or a third weight slot does not
  // fit; tiles whose 64-k stage is too short to cover a trip to HBM (128 x 256:
  // about 0.5 us of MFMA work) get three of each.
  constexpr int kLds2 = (3 * BM + 2 * BN) * kCH * 16, kLds3 = (3 * BM + 3 * BN) * kCH * 16;
  constexpr int NAS = 3;
  constexpr int NBS = (kLds2 > 80 * 1024 && kLds3 <= 160 * 1024) ? 3 : 2;
  constexpr int DA = NAS - 1, DB = NBS - 1;  // prefetch distances in stages
  // Each stage issues its loads for the operand with the shorter distance
  // first (weights on a tie). At the start of stage kt the loads that may
  // still be in flight are those issued after the last one stage kt needs.
  constexpr bool BFIRST = DB <= DA;
  constexpr int WAITN = BFIRST ? (DA == DB ? (DA - 1) * (A_IN + B_IN) : A_IN + (DB - 1) * (A_IN + B_IN))
                               : B_IN + (DA - 1) * (A_IN + B_IN);
  static_assert(NAS >= 2 && NAS <= 3 && NBS >= 2 && NBS <= 3, "ring slots");
  static_assert(WAITN + A_IN + B_IN <= 63, "vmcnt range");
  static_assert((NAS * BM + NBS * BN) * kCH * 16 <= 160 * 1024, "LDS");

  // One array per ring slot, so that reads of one slot are known not to alias
  // the direct loads that fill another; third slots are declared only where used.
  __shared__ u32x4_t A0[BM * kCH], A1[BM * kCH];
  __shared__ u32x4_t B0[BN * kCH], B1[BN * kCH];
  u32x4_t* A2 = A0;
  u32x4_t* B2 = B0;
  if constexpr (NAS == 3) {
    __shared__ u32x4_t A2s[BM * kCH];
    A2 = A2s;
  }
  if constexpr (NBS == 3) {
    __shared__ u32x4_t B2s[BN * kCH];
    B2 = B2s;
  }

  // XCD-aware order. Hardware sends block b to XCD b % 8; give each XCD a
  // contiguous run of logical tiles, ordered (n-tile group of kNG) x (m-tile)
  // x (n-tile in group), so the blocks that run together on one XCD share
  // their token and weight slices in that XCD's L2. The grid is sized for the
  // most m-tiles any grouping can have; the runs are cut from the tiles this
  // grouping has (m-tiles counted from the offsets, and the last group of
  // n-tiles may hold fewer than kNG), so every XCD gets an equal share and the
  // surplus blocks exit at once.
  // n-tiles per group: kTileGroupN, or twice that for the second GEMM on
  // 128-row tiles (measured on the Switch-style layer: 6 % faster; the prefill
  // layer's 256-row tiles are slower with 8 or 16)
  constexpr int kNG = (!G1 && !WGRAD && BM == 128) ? 2 * kTileGroupN : kTileGroupN;
  const int n_nt = (p.N + NCOLS - 1) / NCOLS;
  WaveTiles wt{};
  if constexpr (!WGRAD) wt = wave_tiles(p.offsets, p.E, p.S, p.cap, BM);
  const int n_mt = WGRAD ? p.n_mt : min(p.n_mt, wt.total);
  const int n_t = n_nt * n_mt;
  const int per_xcd = (n_t + 7) / 8;
  const int xi = static_cast<int>(blockIdx.x / 8);
  if (xi >= per_xcd) return;
  const int t = static_cast<int>(blockIdx.x % 8) * per_xcd + xi;
  if (t >= n_t) return;
  // logical tile t -> (n-tile group g of up to kNG n-tiles, m-tile, n-tile in group)
  const int g = t / (kNG * n_mt);
  const int gs = min(kNG, n_nt - g * kNG);
  const int rem = t - g * kNG * n_mt;
  const int mt = rem / gs;
  const int nt = g * kNG + rem % gs;
  int e, row0, rows;
  if constexpr (WGRAD) {  // fixed M rows for every expert: m-tile mt = (expert, tile)
    const int n_mte = (p.M + BM - 1) / BM;
    e = mt / n_mte;
    row0 = (mt % n_mte) * BM;
    rows = min(BM, p.M - row0);
    if (e >= p.E) return;
  } else {
    wave_tile_owner(wt, BM, mt, &e, &row0, &rows);
  }
  const int n0 = nt * NCOLS;

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform: LDS bases stay scalar
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

  // Direct-load sources. Wave wid, instruction u fills chunk slots
  // [(wid*IN + u)*64, +64): row (wid*IN + u)*8 + lane/8, physical chunk
  // lane%8, i.e. logical chunk (lane%8) ^ swz_key(row). Byte offsets are
  // 32-bit: the host keeps every operand matrix at or below 2^32 - 2^23 bytes
  // and d, width at or below 2^20, so row offset + k offset never wraps.
  // Forward GEMMs reduce over k = 0 .. Kd-1 of rows of length Kd; G_WGRAD
  // over expert e's padded range of rows of length ldk, a whole number of
  // stages (so its last stage needs no zero fill).
  const int stride = WGRAD ? p.ldk : Kd;
  const int kb = WGRAD ? p.kofs[e] : 0;
  const int nk = WGRAD ? (p.kofs[e + 1] - kb) / kBK : (Kd + kBK - 1) / kBK;
  const int k_last = WGRAD ? (1 << 30) : (nk - 1) * kBK;  // first k of the last stage
  const uint32_t a_bytes = static_cast<uint32_t>(WGRAD ? p.M : p.x_nrows) * static_cast<uint32_t>(stride) * 2u;
  const uint32_t b_bytes = static_cast<uint32_t>(N) * static_cast<uint32_t>(stride) * 2u;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.x, a_bytes);
  const __amdgpu_buffer_rsrc_t rb1 = buffer_rsrc(p.B + (WGRAD ? size_t{0} : static_cast<size_t>(e) * N * Kd), b_bytes);
  const __amdgpu_buffer_rsrc_t rb3 =
      (NMAT == 2) ? buffer_rsrc(p.B3 + static_cast<size_t>(e) * N * Kd, b_bytes) : rb1;
  // per lane: offset for every stage, and for the last one (out of range past the end of k)
  uint32_t a_vo[A_IN], a_vl[A_IN], b_vo[B_IN], b_vl[B_IN];
#pragma unroll
  for (int u = 0; u < A_IN; ++u) {
    const int r = (wid * A_IN + u) * kRPI + lane / kCH;
    const int kc = ((lane % kCH) ^ swz_key(r)) * 8;
    const int s = row0 + min(r, rows - 1);
    const int src_row = (p.x_rows != nullptr) ? p.x_rows[s] : s;
    a_vo[u] = (static_cast<uint32_t>(src_row) * static_cast<uint32_t>(stride) + static_cast<uint32_t>(kc)) * 2u;
    a_vl[u] = (WGRAD || k_last + kc < Kd) ? a_vo[u] : a_bytes;
  }
#pragma unroll
  for (int u = 0; u < B_IN; ++u) {
    int mat;
    const int r = (wid * B_IN + u) * kRPI + lane / kCH;
    const int kc = ((lane % kCH) ^ swz_key(r)) * 8;
    const int n = min(brow_col(r, &mat), N - 1);
    b_vo[u] = (static_cast<uint32_t>(n) * static_cast<uint32_t>(stride) + static_cast<uint32_t>(kc)) * 2u;
    b_vl[u] = (WGRAD || k_last + kc < Kd) ? b_vo[u] : b_bytes;
  }
  // Load u of the token rows of the stage starting at k0.
  auto load_a = [&](int u, int k0, u32x4_t* As) {
    lds_load16(ra, k0 >= k_last ? a_vl[u] : a_vo[u], (kb + min(k0, k_last)) * 2, As + (wid * A_IN + u) * 64);
  };
  auto load_b = [&](int u, int k0, u32x4_t* Bs) {
    int mat;
    (void)brow_col((wid * B_IN + u) * kRPI, &mat);  // the 8 rows of one instruction share a matrix
    lds_load16((NMAT == 2 && mat) ? rb3 : rb1, k0 >= k_last ? b_vl[u] : b_vo[u], (kb + min(k0, k_last)) * 2,
               Bs + (wid * B_IN + u) * 64);
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

  // 256 x 256 tiles on 8 waves (two per SIMD): a wave issuing its MFMA batch
  // runs at raised priority, so the SIMD's other wave does not take the issue
  // slots between its MFMAs (measured: first GEMM of the prefill layer 3 %
  // faster; slower with one wave per SIMD and with 128-row tiles).
  constexpr bool kPrio = BM == 256 && BN == 256 && NW == 8;
  // Stage kt: MFMAs on slots (As, Bs); loads of weights (kt+DB) into Bn and of
  // tokens (kt+DA) into An.
  // mf: std::true_type for a wave that holds rows of the tile, std::false_type
  // for one that does not (it only issues its share of the loads and waits).
  auto run_stage = [&](auto mf, int kt, const u32x4_t* As, const u32x4_t* Bs, u32x4_t* Bn, u32x4_t* An) {
    constexpr bool MF = decltype(mf)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAITN));  // this wave's loads for stage kt landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                   // ... and every wave's
    asm volatile("" ::: "memory");
    bf16x8_t wf[NKS][TN], xf[NKS][TM];
    auto read = [&](int ks) {
      const int c = ks * 2 + fsub;
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[ks][j] = as_bf16x8(Bs[swz(wn * WTN + j * 32 + frow, c)]);
#pragma unroll
      for (int i = 0; i < TM; ++i) xf[ks][i] = as_bf16x8(As[swz(wm * WTM + i * 32 + frow, c)]);
    };
    if constexpr (MF) read(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int idx = ks * PER + q;
        if constexpr (BFIRST) {
          if (idx < B_IN) load_b(idx, (kt + DB) * kBK, Bn);
          else if (idx < A_IN + B_IN) load_a(idx - B_IN, (kt + DA) * kBK, An);
        } else {
          if (idx < A_IN) load_a(idx, (kt + DA) * kBK, An);
          else if (idx < A_IN + B_IN) load_b(idx - A_IN, (kt + DB) * kBK, Bn);
        }
      }
      asm volatile("" ::: "memory");  // keep the loads ahead of the later fragment reads
      if constexpr (MF) {
        if (ks + 1 < NKS) read(ks + 1);
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][j], xf[ks][i], acc[j][i], 0, 0, 0);
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      }
    }
  };

  u32x4_t* const as[3] = {A0, A1, A2};
  u32x4_t* const bs[3] = {B0, B1, B2};
  // Prologue: the loads of virtual stages -max(DA, DB) .. -1, in stage order
  // (those for stages >= 0 only), so that every stage wait counts the same.
#pragma unroll
  for (int j = -(DA > DB ? DA : DB); j < 0; ++j) {
    if (BFIRST && j + DB >= 0) {
#pragma unroll
      for (int u = 0; u < B_IN; ++u) load_b(u, (j + DB) * kBK, bs[(j + DB) % NBS]);
    }
    if (j + DA >= 0) {
#pragma unroll
      for (int u = 0; u < A_IN; ++u) load_a(u, (j + DA) * kBK, as[(j + DA) % NAS]);
    }
    if (!BFIRST && j + DB >= 0) {
#pragma unroll
      for (int u = 0; u < B_IN; ++u) load_b(u, (j + DB) * kBK, bs[(j + DB) % NBS]);
    }
  }
  // Straight-line ring over lcm(NAS, NBS) stages: no merge point for acc inside
  // the loop. Stage i uses token slot i % NAS and weight slot i % NBS and fills
  // token slot (i + DA) % NAS and weight slot (i + DB) % NBS.
  constexpr int RING = NAS == NBS ? NAS : NAS * NBS;
  auto ring = [&](auto mf) {
    int kt = 0;
    for (; kt + RING <= nk; kt += RING) {
#pragma unroll
      for (int i = 0; i < RING; ++i)
        run_stage(mf, kt + i, as[i % NAS], bs[i % NBS], bs[(i + DB) % NBS], as[(i + DA) % NAS]);
    }
#pragma unroll
    for (int i = 0; i + 1 < RING; ++i)
      if (kt + i < nk) run_stage(mf, kt + i, as[i % NAS], bs[i % NBS], bs[(i + DB) % NBS], as[(i + DA) % NAS]);
  };
  // A tile with few rows (a small expert, the last tile of a group) leaves the
  // waves past its rows without work: they skip the fragment reads and MFMAs
  // (wave-uniform choice, once per tile).
  if (wm * WTM < rows) ring(std::true_type{});
  else ring(std::false_type{});
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in LDS after the block ends
  asm volatile("" ::: "memory");

  // Epilogue. Accumulator (j, i), register r: token = i*32 + lane%32 of the
  // wave's rows; weight row = j*32 + (r/4)*8 + (lane/32)*4 + r%4.
  constexpr int TNO = TN / NMAT;  // output column tiles per wave
  constexpr bool DZ = (MODE == G2_DZ_SWIGLU || MODE == G2_DZ_GELU);
  // gate-gradient terms of a row: column tiles j hold columns j*32 .. j*32+31
  // of the wave's WTN, so 64-column block b is j = 2b, 2b+1 (both lane halves)
  constexpr int NDB = DZ ? (WTN + kDgpCols - 1) / kDgpCols : 1;
  static_assert(!DZ || WTN % kDgpCols == 0, "dZ column blocks");
  float dgs[TM][NDB];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int b = 0; b < NDB; ++b) dgs[i][b] = 0.0f;
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
        if constexpr (MODE == G1_SWIGLU_Z) {  // x W1 | x W3 side by side, rows of 2N; and a
          float z1[4], z3[4], av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            z1[q] = acc[j][i][g * 4 + q];
            z3[q] = acc[j + TNO][i][g * 4 + q];
            av[q] = silu(z1[q]) * z3[q];
          }
          bf16_t* row = static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * 2 * N;
          *reinterpret_cast<u32x2_t*>(row + n) = u32x2_t{pack_bf16x2(z1[0], z1[1]), pack_bf16x2(z1[2], z1[3])};
          *reinterpret_cast<u32x2_t*>(row + N + n) =
              u32x2_t{pack_bf16x2(z3[0], z3[1]), pack_bf16x2(z3[2], z3[3])};
          *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out_act) + static_cast<size_t>(s) * N + n) =
              u32x2_t{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
          continue;
        }
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
        if constexpr (DZ) {  // v = u: gate-gradient terms a u, then dA = g u
          const u32x2_t ap = *reinterpret_cast<const u32x2_t*>(p.ain + static_cast<size_t>(s) * N + n);
          const uint32_t aw[2] = {ap[0], ap[1]};
          const float gs = p.rgate[s];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float av = __uint_as_float(q % 2 ? (aw[q / 2] & 0xFFFF0000u) : (aw[q / 2] << 16));
            dgs[i][(j * 32) / kDgpCols] = fmaf(av, v[q], dgs[i][(j * 32) / kDgpCols]);
            v[q] *= gs;
          }
        }
        if (MODE == G1_SWIGLU || MODE == G1_GELU || MODE == G1_GELU_Z) {
          *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if (MODE == G1_GELU_Z) {
            *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out_act) + static_cast<size_t>(s) * N + n) =
                u32x2_t{pack_bf16x2(gelu_exact(v[0]), gelu_exact(v[1])),
                        pack_bf16x2(gelu_exact(v[2]), gelu_exact(v[3]))};
          }
        } else if (MODE == G2_DZ_SWIGLU) {  // v = dA; dz1 = dA z3 silu'(z1), dz3 = dA silu(z1)
          const bf16_t* zr = p.zin + static_cast<size_t>(s) * 2 * N;
          const u32x2_t z1p = *reinterpret_cast<const u32x2_t*>(zr + n);
          const u32x2_t z3p = *reinterpret_cast<const u32x2_t*>(zr + N + n);
          const uint32_t z1w[2] = {z1p[0], z1p[1]}, z3w[2] = {z3p[0], z3p[1]};
          float d1[4], d3[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a1 = z1w[q / 2], a3 = z3w[q / 2];
            const float z1 = __uint_as_float(q % 2 ? (a1 & 0xFFFF0000u) : (a1 << 16));
            const float z3 = __uint_as_float(q % 2 ? (a3 & 0xFFFF0000u) : (a3 << 16));
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z1 * -1.4426950408889634f));
            d1[q] = v[q] * z3 * (sg * (1.0f + z1 * (1.0f - sg)));
            d3[q] = v[q] * (z1 * sg);
          }
          bf16_t* orow = static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * 2 * N;
          *reinterpret_cast<u32x2_t*>(orow + n) = u32x2_t{pack_bf16x2(d1[0], d1[1]), pack_bf16x2(d1[2], d1[3])};
          *reinterpret_cast<u32x2_t*>(orow + N + n) = u32x2_t{pack_bf16x2(d3[0], d3[1]), pack_bf16x2(d3[2], d3[3])};
        } else if (MODE == G2_DZ_GELU) {  // dz = dA gelu'(z)
          const u32x2_t zp = *reinterpret_cast<const u32x2_t*>(p.zin + static_cast<size_t>(s) * N + n);
          const uint32_t zw[2] = {zp[0], zp[1]};
          float dz[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a = zw[q / 2];
            const float x = __uint_as_float(q % 2 ? (a & 0xFFFF0000u) : (a << 16));
            const float gp = 0.5f * (1.0f + erff(x * 0.70710678118654752440f)) +
                             x * expf(-0.5f * x * x) * 0.39894228040143267794f;
            dz[q] = v[q] * gp;
          }
          *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n) =
              u32x2_t{pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3])};
        } else if (MODE == G_WGRAD) {
          float* dst = s < p.split
                           ? static_cast<float*>(p.out) + (static_cast<size_t>(e) * p.split + s) * N + n
                           : p.out2 + (static_cast<size_t>(e) * (p.M - p.split) + (s - p.split)) * N + n;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
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
  if constexpr (DZ) {
    // lanes l and l ^ 32 hold the same rows: add the other half's columns
    // (lower half first), then lanes 0..31 store one row each per block
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const float other = __shfl_xor(dgs[i][b], 32);
        dgs[i][b] = lane < 32 ? dgs[i][b] + other : other + dgs[i][b];
      }
    if (lane < 32) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rl = wm * WTM + i * 32 + lane;
        if (rl >= rows) continue;
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          const int c0 = n0 + wn * WTN + b * kDgpCols;
          if (c0 < N) p.dgp[static_cast<size_t>(c0 / kDgpCols) * p.S + row0 + rl] = dgs[i][b];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- streaming kernel

constexpr int kStreamWaves = 4;

// KU: k per step = KU runs of 32 contiguous k (8 per lane group) per row.
template <int MODE, int NR, int MC, int NBUF, int KU>
__global__ __launch_bounds__(kStreamWaves * 64) void gemm_stream_kernel(GemmParams p, int n_groups) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  constexpr int kKS = KU * 32;
  const int e = blockIdx.x / n_groups;
  const int grp = blockIdx.x % n_groups;
  int beg, end_row;
  expert_rows(p.offsets, e, p.S, p.cap, &beg, &end_row);
  const int rows = min(end_row - beg, MC * 16);  // the host guarantees <= MC * 16 rows per expert
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

  u32x4_t wreg[NBUF][NMAT][NR][KU];
  u32x4_t xreg[NBUF][MC][KU];
  auto load = [&](int slot, int k0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
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
    for (int u = 0; u < KU; ++u)
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
  if constexpr (NBUF == 2) {
    // explicit register double buffer: one k-step in flight per wave
    load(0, 0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      load(1, (kt + 1) * kKS);
      compute(0);
      if (kt + 2 < nk) load(0, (kt + 2) * kKS);
      compute(1);
    }
    if (kt < nk) compute(0);
  } else {
    // single buffer: fewer registers, more waves per SIMD to keep loads in flight
    for (int kt = 0; kt < nk; ++kt) {
      load(0, kt * kKS);
      compute(0);
    }
  }

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
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  p.n_mt = MODE == G_WGRAD ? p.E * ((p.M + BM - 1) / BM) : (S + BM - 1) / BM + min(p.E, S);
  const int n_nt = (p.N + BN / NMAT - 1) / (BN / NMAT);
  const size_t total = static_cast<size_t>(n_nt) * p.n_mt;
  const size_t grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, WN, MODE>), dim3(static_cast<unsigned>(grid)),
                     dim3(WM * WN * 64), 0, st, p);
  return hipGetLastError();
}

// Tile shape from the mean rows per expert (S / E): with about 1k rows per
// expert, 256 x 256 tiles (the fewest bytes moved per flop) on 8 waves, two per
// SIMD, so that one wave's MFMAs run while the other waits. The backward's dZ
// GEMM (derivative of the activation in the epilogue) runs them on 4 waves of
// 128 x 128, which read a third fewer LDS bytes per MFMA and hold their
// accumulators in the AGPRs (measured: 8 waves 5 % slower there; on the
// forward second GEMM 4 waves were 5 % faster until the 8-wave kernel raised
// its priority around the MFMAs, now 8 waves are 2 % faster). With about 100
// rows per expert, 128 x 256 tiles on 8 waves with the weights two stages
// ahead (measured on the Switch-style layer: 21 % faster than one stage ahead
// on the first GEMM; on the second 5 % faster than 128 x 128 tiles at two
// blocks per CU). Small grids fall back to 128 x 128 so that the chip is
// still covered.
template <int MODE>
hipError_t launch_tile_auto(GemmParams p, int S, hipStream_t st) {
  constexpr bool G1 = (MODE == G1_SWIGLU || MODE == G1_GELU || MODE == G1_SWIGLU_Z || MODE == G1_GELU_Z);
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  const int mean_rows = S / max(p.E, 1);
  auto blocks = [&](int bm, int bn) {
    return static_cast<long>((S + bm - 1) / bm + min(p.E, S)) * ((p.N + bn / NMAT - 1) / (bn / NMAT));
  };
  if (mean_rows >= 512 && blocks(256, 256) >= 2 * 256) {
    return (G1 || MODE == G2_OPERM || MODE == G2_FUSED_Y) ? launch_tile<256, 256, 4, 2, MODE>(p, S, st)
                                                          : launch_tile<256, 256, 2, 2, MODE>(p, S, st);
  }
  if (blocks(128, 256) >= 2 * 256) return launch_tile<128, 256, 4, 2, MODE>(p, S, st);
  return launch_tile<128, 128, 2, 2, MODE>(p, S, st);
}

template <int MODE, int NR, int NBUF, int KU>
hipError_t launch_stream(GemmParams p, int max_rows, hipStream_t st) {
  const int n_groups = (p.N + kStreamWaves * NR * 16 - 1) / (kStreamWaves * NR * 16);
  const dim3 grid(static_cast<unsigned>(p.E * n_groups));
  if (max_rows <= 16) {
    hipLaunchKernelGGL((gemm_stream_kernel<MODE, NR, 1, NBUF, KU>), grid, dim3(kStreamWaves * 64), 0, st, p,
                       n_groups);
  } else {
    hipLaunchKernelGGL((gemm_stream_kernel<MODE, NR, 2, NBUF, KU>), grid, dim3(kStreamWaves * 64), 0, st, p,
                       n_groups);
  }
  return hipGetLastError();
}

constexpr int kStreamMaxRows = 32;
// Measured on the Mixtral-shaped decode layer: one 16-row weight fragment per
// wave, with a register double buffer of 64-k steps for GEMM1 (96 registers:
// five waves per SIMD, so its 7168 waves run in 1.4 rounds; 128-k steps took 144
// registers and 2.3 rounds and were 1.5 % slower, 32-k steps no faster) and a
// single buffer of 128-k steps (more waves per SIMD) for GEMM2.
constexpr int kStreamNR1 = 1, kStreamBuf1 = 2, kStreamKU1 = 2;  // fragments per wave, buffers, 32-k runs per step
constexpr int kStreamNR2 = 1, kStreamBuf2 = 1, kStreamKU2 = 4;

}  // namespace

hipError_t launch_gemm1_bf16(const FfnArgs& f, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(f.x);
  p.x_rows = f.x_rows;
  p.x_nrows = f.x_rows != nullptr ? f.S / f.K : f.S;
  p.cap = f.cap;
  p.offsets = f.offsets;
  p.B = static_cast<const bf16_t*>(f.W1);
  p.B3 = static_cast<const bf16_t*>(f.W3);
  p.bias = static_cast<const bf16_t*>(f.b1);
  p.out = f.a;
  p.E = f.E;
  p.N = f.width;
  p.Kd = f.d;
  p.S = f.S;
  const bool swiglu = f.act == 1;
  if (f.max_rows_per_expert <= kStreamMaxRows) {
    return swiglu ? launch_stream<G1_SWIGLU, kStreamNR1, kStreamBuf1, kStreamKU1>(p, f.max_rows_per_expert, st)
                  : launch_stream<G1_GELU, kStreamNR1, kStreamBuf1, kStreamKU1>(p, f.max_rows_per_expert, st);
  }
  return swiglu ? launch_tile_auto<G1_SWIGLU>(p, f.S, st) : launch_tile_auto<G1_GELU>(p, f.S, st);
}

hipError_t launch_gemm2_bf16(const FfnArgs& f, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(f.a);
  p.x_nrows = f.S;
  p.cap = f.cap;
  p.offsets = f.offsets;
  p.B = static_cast<const bf16_t*>(f.W2);
  p.B3 = nullptr;
  p.bias = static_cast<const bf16_t*>(f.b2);
  p.E = f.E;
  p.N = f.d;
  p.Kd = f.width;
  p.S = f.S;
  if (f.fused_y) {
    p.out = f.y;
    p.slot_token = f.slot_token;
    p.gate = f.topk_gate;
  } else {
    p.out = f.o_perm;
  }
  if (f.max_rows_per_expert <= kStreamMaxRows) {
    return f.fused_y ? launch_stream<G2_FUSED_Y, kStreamNR2, kStreamBuf2, kStreamKU2>(p, f.max_rows_per_expert, st)
                     : launch_stream<G2_OPERM, kStreamNR2, kStreamBuf2, kStreamKU2>(p, f.max_rows_per_expert, st);
  }
  return f.fused_y ? launch_tile_auto<G2_FUSED_Y>(p, f.S, st) : launch_tile_auto<G2_OPERM>(p, f.S, st);
}

}  // namespace moe

// ---------------------------------------------------------------------------- backward pass GEMMs

namespace moe {

hipError_t launch_bwd_z_bf16(const FfnArgs& f, void* z, void* a, hipStream_t st) {
  GemmParams p{};
  p.out_act = a;
  p.x = static_cast<const bf16_t*>(f.x);
  p.x_rows = f.x_rows;
  p.x_nrows = f.x_rows != nullptr ? f.S / f.K : f.S;
  p.cap = f.cap;
  p.offsets = f.offsets;
  p.B = static_cast<const bf16_t*>(f.W1);
  p.B3 = static_cast<const bf16_t*>(f.W3);
  p.bias = static_cast<const bf16_t*>(f.b1);
  p.out = z;
  p.E = f.E;
  p.N = f.width;
  p.Kd = f.d;
  p.S = f.S;
  return f.act == 1 ? launch_tile_auto<G1_SWIGLU_Z>(p, f.S, st) : launch_tile_auto<G1_GELU_Z>(p, f.S, st);
}

hipError_t launch_bwd_grouped_bf16(const void* x, int S, const int32_t* offsets, int cap, int E, const void* B,
                                   const void* bias, int N, int Kd, float* out, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(x);
  p.bias = static_cast<const bf16_t*>(bias);
  p.x_nrows = S;
  p.cap = cap;
  p.offsets = offsets;
  p.B = static_cast<const bf16_t*>(B);
  p.out = out;
  p.E = E;
  p.N = N;
  p.Kd = Kd;
  p.S = S;
  return launch_tile_auto<G2_OPERM>(p, S, st);
}

hipError_t launch_bwd_dz_bf16(const void* dy, int T, const int32_t* slot_token, int S, const int32_t* offsets,
                              int cap, int E, const void* W2T, int N, int Kd, const void* z, int act,
                              const float* rgate, const void* a, float* dgp, void* dZ, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(dy);
  p.x_rows = slot_token;
  p.x_nrows = T;
  p.cap = cap;
  p.offsets = offsets;
  p.B = static_cast<const bf16_t*>(W2T);
  p.zin = static_cast<const bf16_t*>(z);
  p.rgate = rgate;
  p.ain = static_cast<const bf16_t*>(a);
  p.dgp = dgp;
  p.out = dZ;
  p.E = E;
  p.N = N;
  p.Kd = Kd;
  p.S = S;
  return act == 1 ? launch_tile_auto<G2_DZ_SWIGLU>(p, S, st) : launch_tile_auto<G2_DZ_GELU>(p, S, st);
}

hipError_t launch_bwd_wgrad_bf16(const void* A, int M, const void* B, int N, int ldk, const int32_t* kofs, int E,
                                 float* out, float* out2, int split, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(A);
  p.B = static_cast<const bf16_t*>(B);
  p.kofs = kofs;
  p.M = M;
  p.ldk = ldk;
  p.split = split;
  p.out = out;
  p.out2 = out2;
  p.E = E;
  p.N = N;
  p.Kd = ldk;
  return launch_tile<256, 256, 4, 2, G_WGRAD>(p, 0, st);
}

}  // namespace moe

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
//  * gemm_slab_kernel (rows per expert <= 32): every wave streams slabs of 16
//    weight rows over the whole reduction with v_mfma_f32_16x16x32_bf16, the
//    weights as the M operand and up to 32 token rows as N; weights are read
//    from HBM exactly once, which is what bounds decode-sized batches.
#include <algorithm>
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
  // Weights stored with k as the row index (gemm_tile_kernel<..., BT = true>):
  // B is [E][Kd1][N] with N contiguous, Kd1 = kb3 > 0 rows of B followed by
  // kb3 rows of B3 (the SwiGLU input gradient dZ [W1; W3]), or Kd1 = Kd.
  int kb3;
  // G2_OPERM with split tails (gemm_tile_kernel<..., TS = true>): an expert's
  // last m-tile of at most BM / WM rows is computed as ks tiles, part j over
  // stages [j q, (j + 1) q) of the reduction (q = ceil(stages / ks)); part j
  // writes its rows r (0 .. 63) to tail_part[(j E + e) 64 + r][N] (float32,
  // the bias in part 0), which tail_sum_kernel adds into o_perm.
  float* tail_part;
  int ks;
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

// Weights stored with k as the row index (the backward pass reads W2 and
// [W1; W3] this way, as stored for the forward pass): a weight slot holds 64
// rows k of BN columns, 16-byte chunk c of row k at c ^ bt_key(k). An MFMA
// fragment (32 columns x 16 k; lane l: column l % 32, k 8 (l / 32) .. + 7) is
// two ds_read_b64_tr_b16. That instruction works on groups of 16 lanes:
// element j of lane i of a group is element i % 4 of the 8 bytes lane
// 4 j + i / 4 addresses (lane layout checked on the hardware). So lane
// s = 16 G + 4 j + q addresses row 8 (G / 2) + 4 r + j, columns
// 16 (G % 2) + 4 q .. + 3 of the fragment, and read r = 0, 1 delivers the
// fragment's k 8 (l / 32) + 4 r .. + 3. With the XOR key, the 16 (row, chunk)
// pairs of either half-wave of a read fall in distinct 16-byte bank groups.
template <int BN> constexpr int kBtCPR = BN / 8;          // chunks per row
template <int BN> constexpr int kBtRows = 64 / (BN / 8);  // rows per direct-load instruction
__device__ __forceinline__ int bt_key(int k) { return 4 * (k & 3); }

template <int BN>
__device__ __forceinline__ int bt_lane_offset(int lane, int col0) {
  const int G = lane / 16, j = (lane % 16) / 4, q = lane % 4;
  const int k = 8 * (G / 2) + j;
  const int c = col0 / 8 + 2 * (G % 2) + q / 2;
  return k * BN * 2 + (c ^ bt_key(k)) * 16 + (q % 2) * 8;
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t bt_fragment(const u32x4_t* slot, int off, int row_bytes) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const char* base = reinterpret_cast<const char*>(slot);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off + 4 * row_bytes));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

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
// ... for vmcnt <= n and for every LDS and scalar memory access (lgkmcnt 0).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// BT: the weight operand stored with k as the row index (forward-style modes:
// [E][Kd][N] per expert; G_WGRAD: [S][N], rows = grouped slots). XT (G_WGRAD
// only): the x operand stored [S][M] with the grouped slots as rows; each
// expert's reduction then runs over its own slots [beg, end) (expert_rows),
// rows past end reading zeros.
template <int BM, int BN, int WM, int WN, int MODE, bool BT = false, bool XT = false, bool PERSIST = false,
          bool TS = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  static_assert(!BT || NMAT == 1, "k-major weights: single-matrix modes");
  static_assert(!XT || MODE == G_WGRAD, "k-major x: weight-gradient GEMMs");
  static_assert(!TS || (MODE == G2_OPERM && !PERSIST), "split tails: second GEMM or dX GEMM into float32 rows");
  static_assert(MODE != G_WGRAD || !BT || XT, "k-major weights of a weight-gradient GEMM need k-major x");
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
  const int ks = TS ? p.ks : 1;
  if constexpr (!WGRAD) wt = wave_tiles(p.offsets, p.E, p.S, p.cap, BM, ks, WTM);
  // wave-uniform values kept in scalar registers (a lane shuffle's result is
  // not known to be uniform, and the persistent tile loop branches on them)
  const int n_mt = __builtin_amdgcn_readfirstlane(WGRAD ? p.n_mt : min(p.n_mt, wt.total));
  const int n_t = n_nt * n_mt;
  const int per_xcd = (n_t + 7) / 8;
  const int xi = static_cast<int>(blockIdx.x / 8);
  if (xi >= per_xcd) return;
  // PERSIST: the grid holds one block per CU (a multiple of 8, so every XCD
  // gets gridDim.x / 8 of them); the block at index xi of its XCD takes the
  // tiles xi, xi + gridDim.x / 8, ... of that XCD's run, and issues the first
  // loads of its next tile before the epilogue of the current one.
  const int t_end = min(n_t, (static_cast<int>(blockIdx.x % 8) + 1) * per_xcd);
  int t = static_cast<int>(blockIdx.x % 8) * per_xcd + xi;
  if (t >= t_end) return;
  int e = 0, row0 = 0, rows = 0, n0 = 0, split = -1;
  // logical tile tt -> (n-tile group g of up to kNG n-tiles, m-tile, n-tile in
  // group) -> expert, rows, first output column; false for a tile past the
  // last expert (weight-gradient grids)
  auto decode = [&](int tt) {
    const int g = tt / (kNG * n_mt);
    const int gs = min(kNG, n_nt - g * kNG);
    const int rem = tt - g * kNG * n_mt;
    const int mt = rem / gs;
    const int ntl = g * kNG + rem % gs;
    n0 = ntl * NCOLS;
    if constexpr (WGRAD) {  // fixed M rows for every expert: m-tile mt = (expert, tile)
      const int n_mte = (p.M + BM - 1) / BM;
      e = mt / n_mte;
      row0 = (mt % n_mte) * BM;
      rows = min(BM, p.M - row0);
      return e < p.E;
    } else {
      wave_tile_owner(wt, BM, mt, &e, &row0, &rows, ks, WTM, &split);
      e = __builtin_amdgcn_readfirstlane(e);
      split = __builtin_amdgcn_readfirstlane(split);
      row0 = __builtin_amdgcn_readfirstlane(row0);
      rows = __builtin_amdgcn_readfirstlane(rows);
      return true;
    }
  };
  if (!decode(t)) return;

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
  // per tile: k range (weight-gradient GEMMs), buffers and per-lane offsets
  int kb = 0, nk = 0, kbeg = 0, kend = 0, k_last = 0;
  const uint32_t a_bytes = XT ? static_cast<uint32_t>(p.S) * static_cast<uint32_t>(p.M) * 2u
                              : static_cast<uint32_t>(WGRAD ? p.M : p.x_nrows) * static_cast<uint32_t>(stride) * 2u;
  const uint32_t b_bytes = static_cast<uint32_t>(N) * static_cast<uint32_t>(stride) * 2u;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.x, a_bytes);
  // k-major weights: Kd1 rows of B per expert (then as many of B3)
  const int Kd1 = (BT && p.kb3 > 0) ? p.kb3 : Kd;
  const uint32_t bt_bytes = static_cast<uint32_t>(WGRAD ? p.S : Kd1) * static_cast<uint32_t>(N) * 2u;
  __amdgpu_buffer_rsrc_t rb1 = ra, rb3 = ra;
  // per lane: offset for every stage, and for the last one (out of range past the end of k)
  uint32_t a_vo[A_IN], a_vl[A_IN], b_vo[B_IN], b_vl[B_IN];
  auto setup = [&]() {
  kb = WGRAD ? p.kofs[e] : 0;
  nk = WGRAD ? (p.kofs[e + 1] - kb) / kBK : (Kd + kBK - 1) / kBK;
  if (TS && split >= 0) {  // one part of the reduction (the host keeps every part non-empty)
    const int q = (nk + ks - 1) / ks;
    kb = split * q * kBK;
    nk = min(q, nk - split * q);
  }
  // k-major weight-gradient operands: expert e's grouped slots (the same
  // count of stages as its padded range kofs[e] .. kofs[e+1])
  if constexpr (XT) expert_rows(p.offsets, e, p.S, p.cap, &kbeg, &kend);
  k_last = WGRAD ? (1 << 30) : (nk - 1) * kBK;  // first k of the last stage
  rb1 = BT ? buffer_rsrc(p.B + (WGRAD ? size_t{0} : static_cast<size_t>(e) * Kd1 * N), bt_bytes)
           : buffer_rsrc(p.B + (WGRAD ? size_t{0} : static_cast<size_t>(e) * N * Kd), b_bytes);
  rb3 = (NMAT == 2) ? buffer_rsrc(p.B3 + static_cast<size_t>(e) * N * Kd, b_bytes)
                    : ((BT && p.kb3 > 0) ? buffer_rsrc(p.B3 + static_cast<size_t>(e) * Kd1 * N, bt_bytes) : rb1);
#pragma unroll
  for (int u = 0; u < A_IN; ++u) {
    if constexpr (XT) {  // the slot layout of k-major weights, over the block's M columns
      const int lr = lane / kBtCPR<BM>;
      const int r = (wid * A_IN + u) * kBtRows<BM> + lr;
      const int gc = (lane % kBtCPR<BM>) ^ bt_key(r);
      const int m = min(row0 + gc * 8, p.M - 8);
      a_vo[u] = (static_cast<uint32_t>(lr) * static_cast<uint32_t>(p.M) + static_cast<uint32_t>(m)) * 2u;
      a_vl[u] = a_vo[u];
    } else {
      const int r = (wid * A_IN + u) * kRPI + lane / kCH;
      const int kc = ((lane % kCH) ^ swz_key(r)) * 8;
      const int s = row0 + min(r, rows - 1);
      const int src_row = (p.x_rows != nullptr) ? p.x_rows[s] : s;
      a_vo[u] = (static_cast<uint32_t>(src_row) * static_cast<uint32_t>(stride) + static_cast<uint32_t>(kc)) * 2u;
      a_vl[u] = (WGRAD || kb + k_last + kc < Kd) ? a_vo[u] : a_bytes;
    }
  }
#pragma unroll
  for (int u = 0; u < B_IN; ++u) {
    if constexpr (BT) {
      // LDS slot [k][BN] (rows of BN columns, 16-byte chunks): instruction u
      // fills rows (wid * B_IN + u) * RB ..; lane l takes row-in-instruction
      // l / CPR and physical chunk l % CPR, i.e. the global chunk
      // (l % CPR) ^ bt_key(row) of the block's columns (columns past N read a
      // valid chunk whose outputs are never stored).
      const int lr = lane / kBtCPR<BN>;
      const int r = (wid * B_IN + u) * kBtRows<BN> + lr;
      const int gc = (lane % kBtCPR<BN>) ^ bt_key(r);
      const int n = min(n0 + gc * 8, N - 8);
      b_vo[u] = (static_cast<uint32_t>(lr) * static_cast<uint32_t>(N) + static_cast<uint32_t>(n)) * 2u;
      b_vl[u] = b_vo[u];
    } else {
      int mat;
      const int r = (wid * B_IN + u) * kRPI + lane / kCH;
      const int kc = ((lane % kCH) ^ swz_key(r)) * 8;
      const int n = min(brow_col(r, &mat), N - 1);
      b_vo[u] = (static_cast<uint32_t>(n) * static_cast<uint32_t>(stride) + static_cast<uint32_t>(kc)) * 2u;
      b_vl[u] = (WGRAD || kb + k_last + kc < Kd) ? b_vo[u] : b_bytes;
    }
  }
  };
  setup();
  // k-major slot rows: the lane's row kbeg + k0 + (first row of instruction
  // u) + lane / CPR, zeros (an offset past the buffer) at or past kend
  auto kmajor_off = [&](uint32_t vo, int rbase, int lr, uint32_t ld, uint32_t bytes) {
    return kbeg + rbase + lr < kend ? vo + static_cast<uint32_t>(kbeg + rbase) * ld * 2u : bytes;
  };
  // Load u of the token rows of the stage starting at k0.
  auto load_a = [&](int u, int k0, u32x4_t* As) {
    if constexpr (XT) {
      const int rbase = k0 + (wid * A_IN + u) * kBtRows<BM>;
      lds_load16(ra, kmajor_off(a_vo[u], rbase, lane / kBtCPR<BM>, p.M, a_bytes), 0, As + (wid * A_IN + u) * 64);
    } else {
      lds_load16(ra, k0 >= k_last ? a_vl[u] : a_vo[u], (kb + min(k0, k_last)) * 2, As + (wid * A_IN + u) * 64);
    }
  };
  auto load_b = [&](auto nt, int u, int k0, u32x4_t* Bs) {
    if constexpr (BT && WGRAD) {
      const int rbase = k0 + (wid * B_IN + u) * kBtRows<BN>;
      lds_load16(rb1, kmajor_off(b_vo[u], rbase, lane / kBtCPR<BN>, N, bt_bytes), 0, Bs + (wid * B_IN + u) * 64);
    } else if constexpr (BT) {
      // rows kb + k0 + (wid * B_IN + u) * RB .. of the reduction (kb: the first
      // k of a split tail's part, else 0): all in B, all in B3 (Kd1 is a
      // multiple of 8, RB <= 4) or all past Kd (zeros, no traffic)
      const int kr = kb + k0 + (wid * B_IN + u) * kBtRows<BN>;
      const bool second = p.kb3 > 0 && kr >= Kd1;
      // byte offsets below 2^32 (the matrix bytes are); passed on as the same 32 bits
      const uint32_t soff = kr >= Kd ? bt_bytes : static_cast<uint32_t>(second ? kr - Kd1 : kr) * N * 2u;
      lds_load16(second ? rb3 : rb1, b_vo[u], static_cast<int>(soff), Bs + (wid * B_IN + u) * 64);
    } else {
      int mat;
      (void)brow_col((wid * B_IN + u) * kRPI, &mat);  // the 8 rows of one instruction share a matrix
      const uint32_t vo = k0 >= k_last ? b_vl[u] : b_vo[u];
      const int so = (kb + min(k0, k_last)) * 2;
      if constexpr (decltype(nt)::value) {  // weights read once: non-temporal
        __builtin_amdgcn_raw_ptr_buffer_load_lds((NMAT == 2 && mat) ? rb3 : rb1,
                                                 (__attribute__((address_space(3))) void*)(Bs + (wid * B_IN + u) * 64),
                                                 16, static_cast<int>(vo), so, 0, 2);
      } else {
        lds_load16((NMAT == 2 && mat) ? rb3 : rb1, vo, so, Bs + (wid * B_IN + u) * 64);
      }
    }
  };

  f32x16_t acc[TN][TM];  // zeroed at the start of every tile

  const int frow = lane % 32;
  const int fsub = lane / 32;  // which of the two 8-wide k chunks of a 16-k step
  // k-major weight fragments: byte offset in the slot of this lane's first
  // transposed read for fragment j (k-step 0)
  int bt_off[TN], xt_off[TM];
#pragma unroll
  for (int j = 0; j < TN; ++j) bt_off[j] = BT ? bt_lane_offset<BN>(lane, wn * WTN + j * 32) : 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) xt_off[i] = XT ? bt_lane_offset<BM>(lane, wm * WTM + i * 32) : 0;

  // 256 x 256 tiles on 8 waves (two per SIMD): a wave issuing its MFMA batch
  // runs at raised priority, so the SIMD's other wave does not take the issue
  // slots between its MFMAs (measured: first GEMM of the prefill layer 3 %
  // faster; slower with one wave per SIMD and with 128-row tiles).
  constexpr bool kPrio = BM == 256 && BN == 256 && NW == 8;
  // Stage kt: MFMAs on slots (As, Bs); loads of weights (kt+DB) into Bn and of
  // tokens (kt+DA) into An.
  // mf: std::true_type for a wave that holds rows of the tile, std::false_type
  // for one that does not (it only issues its share of the loads and waits).
  // On 128-row tiles the MFMAs of a stage's last 16-k step run after the next
  // stage's barrier and first fragment reads (their fragments are in registers
  // once the wait before that barrier has drained the LDS reads, so the slots
  // they came from may be refilled): they cover the
  // latency of those reads (Switch-style layer, first GEMM 0.366 -> 0.355 ms;
  // on 256 x 256 tiles it was slower: prefill first GEMM 1.676 -> 1.706 ms,
  // second 0.984 -> 1.063 ms). Every accumulator still sees its k steps in
  // the same order.
  constexpr bool kDefer = BM == 128;
  bf16x8_t dwf[TN], dxf[TM];  // fragments of the deferred step
  auto mfma_step = [&](const bf16x8_t* w, const bf16x8_t* x) {
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[j], x[i], acc[j][i], 0, 0, 0);
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
  };
  auto run_stage = [&](auto mf, auto nt, int kt, const u32x4_t* As, const u32x4_t* Bs, u32x4_t* Bn, u32x4_t* An) {
    constexpr bool MF = decltype(mf)::value;
    // This wave's loads for stage kt landed. With deferred MFMAs, also the
    // fragment reads of the previous stage's last step: the barrier lets the
    // other waves refill the slots those reads come from, and the barrier does
    // not wait for LDS reads in flight (left pending, an LDS queue backed up by
    // eight waves' reads could let a refill land first: y then varied from run
    // to run on 128-row tiles).
    __builtin_amdgcn_s_waitcnt(kDefer ? vmcnt_lgkm0_imm(WAITN) : vmcnt_imm(WAITN));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                   // ... and every wave's
    asm volatile("" ::: "memory");
    bf16x8_t wf[NKS][TN], xf[NKS][TM];
    auto read = [&](int ks) {
      const int c = ks * 2 + fsub;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BT) {
          wf[ks][j] = bt_fragment(Bs, bt_off[j] + ks * 16 * BN * 2, BN * 2);
        } else {
          wf[ks][j] = as_bf16x8(Bs[swz(wn * WTN + j * 32 + frow, c)]);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (XT) {
          xf[ks][i] = bt_fragment(As, xt_off[i] + ks * 16 * BM * 2, BM * 2);
        } else {
          xf[ks][i] = as_bf16x8(As[swz(wm * WTM + i * 32 + frow, c)]);
        }
      }
    };
    if constexpr (MF) {
      read(0);
      if (kDefer && kt > 0) mfma_step(dwf, dxf);  // the previous stage's last step
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int idx = ks * PER + q;
        if constexpr (BFIRST) {
          if (idx < B_IN) load_b(nt, idx, (kt + DB) * kBK, Bn);
          else if (idx < A_IN + B_IN) load_a(idx - B_IN, (kt + DA) * kBK, An);
        } else {
          if (idx < A_IN) load_a(idx, (kt + DA) * kBK, An);
          else if (idx < A_IN + B_IN) load_b(nt, idx - A_IN, (kt + DB) * kBK, Bn);
        }
      }
      asm volatile("" ::: "memory");  // keep the loads ahead of the later fragment reads
      if constexpr (MF) {
        if (ks + 1 < NKS) read(ks + 1);
        if (!kDefer || ks + 1 < NKS) {
          mfma_step(wf[ks], xf[ks]);
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) dwf[j] = wf[ks][j];
#pragma unroll
          for (int i = 0; i < TM; ++i) dxf[i] = xf[ks][i];
        }
      }
    }
  };

  u32x4_t* const as[3] = {A0, A1, A2};
  u32x4_t* const bs[3] = {B0, B1, B2};
  // Prologue: the loads of virtual stages -max(DA, DB) .. -1, in stage order
  // (those for stages >= 0 only), so that every stage wait counts the same.
  auto prologue = [&](auto nt) {
#pragma unroll
    for (int j = -(DA > DB ? DA : DB); j < 0; ++j) {
      if (BFIRST && j + DB >= 0) {
#pragma unroll
        for (int u = 0; u < B_IN; ++u) load_b(nt, u, (j + DB) * kBK, bs[(j + DB) % NBS]);
      }
      if (j + DA >= 0) {
#pragma unroll
        for (int u = 0; u < A_IN; ++u) load_a(u, (j + DA) * kBK, as[(j + DA) % NAS]);
      }
      if (!BFIRST && j + DB >= 0) {
#pragma unroll
        for (int u = 0; u < B_IN; ++u) load_b(nt, u, (j + DB) * kBK, bs[(j + DB) % NBS]);
      }
    }
  };
  // Straight-line ring over lcm(NAS, NBS) stages: no merge point for acc inside
  // the loop. Stage i uses token slot i % NAS and weight slot i % NBS and fills
  // token slot (i + DA) % NAS and weight slot (i + DB) % NBS.
  constexpr int RING = NAS == NBS ? NAS : NAS * NBS;
  auto ring = [&](auto mf, auto nt) {
    int kt = 0;
    for (; kt + RING <= nk; kt += RING) {
#pragma unroll
      for (int i = 0; i < RING; ++i)
        run_stage(mf, nt, kt + i, as[i % NAS], bs[i % NBS], bs[(i + DB) % NBS], as[(i + DA) % NAS]);
    }
#pragma unroll
    for (int i = 0; i + 1 < RING; ++i)
      if (kt + i < nk) run_stage(mf, nt, kt + i, as[i % NAS], bs[i % NBS], bs[(i + DB) % NBS], as[(i + DA) % NAS]);
  };
  // A tile with few rows (a small expert, the last tile of a group) leaves the
  // waves past its rows without work: they skip the fragment reads and MFMAs
  // (wave-uniform choice, once per tile).
  auto run = [&](auto nt) {
    if constexpr (!PERSIST) prologue(nt);
    if (wm * WTM < rows) {
      ring(std::true_type{}, nt);
      if constexpr (kDefer) {
        if (nk > 0) mfma_step(dwf, dxf);  // the last stage's last step (none for an empty reduction)
      }
    } else {
      ring(std::false_type{}, nt);
    }
  };
  // On 128-row tiles of the forward first GEMM, the only m-tile of an expert
  // reads its weight slice exactly once: those loads go non-temporal (the
  // streaming read pattern that measured fastest for weight-bound GEMMs), while
  // experts with several m-tiles keep their slices in L2 for the other m-tiles.
  // Measured on the Switch-style layer: first GEMM 0.353 -> 0.327 ms; the second
  // GEMM (weight slices of 704 KB, its activations reused by 16 n-tiles) was
  // slower with it (0.229 -> 0.244 ms), and all-non-temporal weight loads were
  // slower everywhere (first GEMM 0.335 -> 0.366 ms, prefill 1.64 -> 1.79 ms).
  constexpr bool kNtOnce = BM == 128 && BN == 256 && !BT && (MODE == G1_SWIGLU || MODE == G1_GELU);
  static_assert(!PERSIST || !kNtOnce, "persistent tiles use the default weight-load policy");

  // Epilogue of the tile (e, row0, rows, n0). Accumulator (j, i), register r:
  // token = i*32 + lane%32 of the wave's rows; weight row = j*32 + (r/4)*8 +
  // (lane/32)*4 + r%4.
  auto epilogue = [&](const int e, const int row0, const int rows, const int n0, const int split) {
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
  if constexpr (DZ) {
    // Per column tile j: every load of its rows and column groups is issued
    // first (rows and columns past the tile's end clamped into it, so no load
    // sits behind a branch), then the math and the stores. Loads placed after
    // a store would wait for it (the output may alias them as far as the
    // compiler knows), which made every group of four columns two round trips.
    constexpr int ZR = MODE == G2_DZ_SWIGLU ? 2 : 1;  // z row length in units of N
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
      u32x2_t ap[TM][4], z1p[TM][4], z3p[TM][4];
      float gsv[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int s = row0 + min(wm * WTM + i * 32 + (lane % 32), rows - 1);
        gsv[i] = p.rgate[s];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = min(n0 + wn * WTN + j * 32 + g * 8 + (lane / 32) * 4, N - 4);
          ap[i][g] = *reinterpret_cast<const u32x2_t*>(p.ain + static_cast<size_t>(s) * N + n);
          const bf16_t* zr = p.zin + static_cast<size_t>(s) * ZR * N;
          z1p[i][g] = *reinterpret_cast<const u32x2_t*>(zr + n);
          if constexpr (ZR == 2) z3p[i][g] = *reinterpret_cast<const u32x2_t*>(zr + N + n);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rl = wm * WTM + i * 32 + (lane % 32);
        if (rl >= rows) continue;
        const int s = row0 + rl;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WTN + j * 32 + g * 8 + (lane / 32) * 4;
          if (n >= N) continue;  // N % 8 == 0: four columns are all in or all out
          // v = u: gate-gradient terms a u, then dA = g u
          float v[4];
          const uint32_t aw[2] = {ap[i][g][0], ap[i][g][1]};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = acc[j][i][g * 4 + q];
            const float av = __uint_as_float(q % 2 ? (aw[q / 2] & 0xFFFF0000u) : (aw[q / 2] << 16));
            dgs[i][(j * 32) / kDgpCols] = fmaf(av, v[q], dgs[i][(j * 32) / kDgpCols]);
            v[q] *= gsv[i];
          }
          const uint32_t z1w[2] = {z1p[i][g][0], z1p[i][g][1]};
          if constexpr (MODE == G2_DZ_SWIGLU) {  // dz1 = dA z3 silu'(z1), dz3 = dA silu(z1)
            const uint32_t z3w[2] = {z3p[i][g][0], z3p[i][g][1]};
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
            *reinterpret_cast<u32x2_t*>(orow + N + n) =
                u32x2_t{pack_bf16x2(d3[0], d3[1]), pack_bf16x2(d3[2], d3[3])};
          } else {  // dz = dA gelu'(z)
            float dz[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t a = z1w[q / 2];
              const float x = __uint_as_float(q % 2 ? (a & 0xFFFF0000u) : (a << 16));
              const float gp = 0.5f * (1.0f + erff(x * 0.70710678118654752440f)) +
                               x * expf(-0.5f * x * x) * 0.39894228040143267794f;
              dz[q] = v[q] * gp;
            }
            *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n) =
                u32x2_t{pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3])};
          }
        }
      }
    }
  }
  // K = 1 gated scatter: each row's token and gate, loaded once per row
  // (not once per column group, where each would wait for the stores before it)
  int fy_t[TM];
  float fy_g[TM];
  if constexpr (MODE == G2_FUSED_Y) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int s = row0 + min(wm * WTM + i * 32 + (lane % 32), rows - 1);
      fy_t[i] = p.slot_token[s];
      fy_g[i] = p.gate[fy_t[i]];
    }
  }
  // The bias of every column group of the wave, loaded once, 8 bytes per group
  // (four 2-byte loads per group, each after the stores before it, took most
  // of a short reduction's tile).
  constexpr bool BIAS = MODE == G1_GELU || MODE == G1_GELU_Z || MODE == G2_OPERM || MODE == G2_FUSED_Y;
  const bool has_bias = BIAS && p.bias != nullptr && split <= 0;  // split tails: the bias in part 0
  u32x2_t bias4[BIAS ? TNO : 1][4];
  if constexpr (BIAS) {
    if (has_bias) {
#pragma unroll
      for (int j = 0; j < TNO; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = min(n0 + wn * (WTN / NMAT) + j * 32 + g * 8 + (lane / 32) * 4, N - 4);
          bias4[j][g] = *reinterpret_cast<const u32x2_t*>(p.bias + static_cast<size_t>(e) * N + n);
        }
    }
  }
#pragma unroll
  for (int j = 0; j < (DZ ? 0 : TNO); ++j)
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
          float bq = 0.0f;
          if constexpr (BIAS) {
            const uint32_t w = bias4[j][g][q / 2];
            bq = __uint_as_float(q % 2 ? (w & 0xFFFF0000u) : (w << 16));
          }
          if constexpr (MODE == G1_SWIGLU) {
            v[q] = silu(v1) * acc[j + TNO][i][g * 4 + q];
          } else if constexpr (MODE == G1_GELU) {
            v[q] = gelu_exact(has_bias ? v1 + bq : v1);
          } else {
            v[q] = has_bias ? v1 + bq : v1;
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
        } else if (MODE == G_WGRAD) {
          float* dst = s < p.split
                           ? static_cast<float*>(p.out) + (static_cast<size_t>(e) * p.split + s) * N + n
                           : p.out2 + (static_cast<size_t>(e) * (p.M - p.split) + (s - p.split)) * N + n;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else if (MODE == G2_OPERM) {
          float* dst = static_cast<float*>(p.out) + static_cast<size_t>(s) * N + n;
          if (TS && split >= 0) dst = p.tail_part + (static_cast<size_t>(split * p.E + e) * 64 + rl) * N + n;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          const int t = fy_t[i];
          const float gt = fy_g[i];
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
  };

  if constexpr (PERSIST) prologue(std::false_type{});
  for (;;) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
    if constexpr (kNtOnce) {
      if (__shfl(wt.cnt, e) <= BM) run(std::true_type{});
      else run(std::false_type{});
    } else {
      run(std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in LDS after the block ends
    asm volatile("" ::: "memory");
    const int te = e, trow0 = row0, trows = rows, tn0 = n0, tsplit = split;
    bool more = false;
    if constexpr (PERSIST) {
      t += static_cast<int>(gridDim.x / 8);
      more = t < t_end;
      if (more) {
        // every wave has read its last fragments of this tile: the next
        // tile's first stages may go into the slots
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        decode(t);
        setup();
        prologue(std::false_type{});
      }
    }
    epilogue(te, trow0, trows, tn0, tsplit);
    if constexpr (!PERSIST) {
      break;
    } else {
      if (!more) break;
    }
  }
}

// ---------------------------------------------------------------------------- slab kernel
//
// Decode-sized groups (at most MC * 16 rows per expert): the weights are read
// from HBM exactly once and bound the time, so everything is arranged for the
// weight stream. A slab is 16 weight rows (of W1 and W3 for SwiGLU) of one
// hit expert over the whole reduction; slabs of all hit experts are numbered
// expert by expert and wave g of G takes slabs g, g + G, ... (the host sizes
// G so that they divide evenly when every expert is hit), running one
// software pipeline over the stages (64 k) of all its slabs, so no wave waits
// at a slab boundary and none is left over at the end.
// Weights: each stage of a slab is 16 rows x 128 bytes; two non-temporal
// direct-to-LDS loads per matrix, each covering 8 rows with 8 lanes per
// 128-byte line (whole lines per instruction: measured on the Mixtral decode
// weights, 6.85 TB/s against 6.10 for half lines per instruction and plain
// loads). The wave's private LDS ring holds NBUF stages, loaded NBUF - 1
// ahead; the MFMA fragments are read back with the same chunk swizzle as the
// tiled kernel. One wave per block: no barriers.
// Tokens: each stage's token rows (at most MC * 16; cached, reused by every
// slab of the expert) are loaded into the same ring slot, each lane fetching
// exactly the 16 bytes it later reads as its MFMA fragment (rows past the
// expert's count and k past the end read zeros through the range check). No
// load of the loop writes a register, so no compiler-inserted wait drains
// the pipeline (with a register ring for the tokens the compiler waited for
// all loads at the top of the loop). Stages past the wave's last issue the
// same loads at offsets past the end (zeros, no memory traffic), so every
// stage waits for the same count.
// MFMA v_mfma_f32_16x16x32_bf16, weights as the M operand: lane (a = l / 16,
// b = l % 16) reads weight row b and token row b at k chunk 4u + a of the
// stage for the u-th MFMA, so both operands agree on which k a slot holds.
// IDX: how grouped row s finds its row of x. 0: row s itself; 1: x_rows[s],
// with all S <= 256 ids held in four registers per lane and picked by lane
// shuffles (no memory access at a slab switch); 2: x_rows[s] loaded at the
// switch.
constexpr int kSlabRows = 16;
// Ring depth: two stages (one in flight while one is computed), with as many
// waves per CU as the LDS allows (up to 8). Measured on the Mixtral decode
// layer (first / second GEMM): depth 2: 285 / 144 us; 3: 287 / 158 us;
// 4 and 5: 296 / 170 us (with deeper rings the compiler adds waits of its own
// for direct loads into other slots before some fragment reads).
constexpr int kSlabBuf1 = 2;
constexpr int kSlabBuf2 = 2;
constexpr int kSlabIdsMax = 256;

// 16 bytes per lane into LDS, non-temporal (the nt cache-policy bit).
__device__ __forceinline__ void lds_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, u32x4_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16,
                                           static_cast<int>(voff), 0, 0, 2);
}

// Store through a pointer the compiler knows to be global: stores through a
// generic pointer may write LDS, and then every later LDS read waits for them.
template <typename T>
__device__ __forceinline__ void store_global(void* ptr, T v) {
  *(__attribute__((address_space(1))) T*)(ptr) = v;
}

template <int MODE, int MC, int NBUF, int IDX>
__global__ __launch_bounds__(64) void gemm_slab_kernel(GemmParams p) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  constexpr int WSLOT = NMAT * kSlabRows * kCH;   // u32x4 of weights per ring stage
  constexpr int SLOT = WSLOT + MC * 2 * 64;       // + the token fragments (two per 16 rows)
  constexpr int L = 2 * NMAT + 2 * MC;          // loads per stage
  constexpr int WAIT = (NBUF - 1) * L;          // loads that may stay in flight past a stage's own
  static_assert(WAIT <= 63, "vmcnt range");
  static_assert(NBUF >= 2 && NBUF <= 6, "ring depth");
  // One array per ring slot, so that the fragment reads of one slot are known
  // not to alias the direct loads in flight into the others.
  __shared__ u32x4_t R0[SLOT], R1[SLOT];
  u32x4_t *R2p = nullptr, *R3p = nullptr, *R4p = nullptr, *R5p = nullptr;
  if constexpr (NBUF > 2) {
    __shared__ u32x4_t R2[SLOT];
    R2p = R2;
  }
  if constexpr (NBUF > 3) {
    __shared__ u32x4_t R3[SLOT];
    R3p = R3;
  }
  if constexpr (NBUF > 4) {
    __shared__ u32x4_t R4[SLOT];
    R4p = R4;
  }
  if constexpr (NBUF > 5) {
    __shared__ u32x4_t R5[SLOT];
    R5p = R5;
  }
  // (slot is a constant wherever this is called: the loops over slots are unrolled)
  auto ring = [&](int slot) {
    return slot == 0 ? R0 : slot == 1 ? R1 : slot == 2 ? R2p : slot == 3 ? R3p : slot == 4 ? R4p : R5p;
  };
  const int lane = threadIdx.x;
  const int la = lane / 16, lb = lane % 16;
  const int N = p.N, Kd = p.Kd;
  const int G = static_cast<int>(gridDim.x), gw = static_cast<int>(blockIdx.x);

  // hit experts: lane e holds expert e's first row and row count
  int rbeg = 0, rcnt = 0;
  if (lane < p.E) {
    int b, en;
    expert_rows(p.offsets, lane, p.S, p.cap, &b, &en);
    rbeg = b;
    rcnt = min(en - b, MC * 16);  // the host guarantees at most MC * 16 rows per expert
  }
  const uint64_t hit = __ballot(rcnt > 0);
  const int hrank = __popcll(hit & ((uint64_t{1} << lane) - 1));  // rank of this lane among hit experts
  const int nsl = (N + kSlabRows - 1) / kSlabRows;
  const int total = __popcll(hit) * nsl;
  const int my = gw < total ? (total - 1 - gw) / G + 1 : 0;
  if (my == 0) return;
  const int nks = (Kd + kBK - 1) / kBK;
  const int nstage = my * nks;
  int ids[4] = {0, 0, 0, 0};
  if constexpr (IDX == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ids[q] = lane + 64 * q < p.S ? p.x_rows[lane + 64 * q] : 0;
  }

  const uint32_t w_bytes = static_cast<uint32_t>(N) * static_cast<uint32_t>(Kd) * 2u;
  const uint32_t x_bytes = static_cast<uint32_t>(p.x_nrows) * static_cast<uint32_t>(Kd) * 2u;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.x, x_bytes);

  // Slab i of this wave -> expert, first weight row, token rows (wave-uniform).
  struct Slab {
    int e, n0, beg, rows;
  };
  auto slab = [&](int i) {
    const int s = gw + min(i, my - 1) * G;
    const int h = s / nsl;
    Slab r;
    r.e = __ffsll(static_cast<unsigned long long>(__ballot(rcnt > 0 && hrank == h))) - 1;
    r.n0 = (s - h * nsl) * kSlabRows;
    r.beg = __shfl(rbeg, r.e);
    r.rows = __shfl(rcnt, r.e);
    return r;
  };

  // Load side: the slab being loaded and its per-lane offsets.
  // Weight instruction j covers rows 8j .. 8j+7 of the slab: lane l reads row
  // 8j + l / 8, physical chunk l % 8 = logical chunk (l % 8) ^ swz_key(row).
  __amdgpu_buffer_rsrc_t rw[NMAT];
  uint32_t wvo[2];   // byte offset of this lane's weight chunk at k = 0 (or past the end)
  int wkc[2];        // its logical chunk's first k
  uint32_t xvo[MC];  // byte offset of this lane's token row at k = 0 (or past the end)
  int li = 0, lkk = 0;
  auto set_load_slab = [&](const Slab& sl) {
    rw[0] = buffer_rsrc(p.B + static_cast<size_t>(sl.e) * N * Kd, w_bytes);
    if constexpr (NMAT == 2) rw[NMAT - 1] = buffer_rsrc(p.B3 + static_cast<size_t>(sl.e) * N * Kd, w_bytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * j + lane / 8;
      wkc[j] = ((lane % 8) ^ swz_key(r)) * 8;
      const int n = sl.n0 + r;
      wvo[j] = n < N ? (static_cast<uint32_t>(n) * static_cast<uint32_t>(Kd) + static_cast<uint32_t>(wkc[j])) * 2u
                     : w_bytes;
    }
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int r = c * 16 + lb;
      const int s = sl.beg + min(r, sl.rows - 1);  // a grouped row of the expert (rows >= 1)
      int src = s;
      if constexpr (IDX == 1) {
        int v = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = __shfl(ids[q], s & 63);
          if ((s >> 6) == q) v = t;
        }
        src = v;
      } else if constexpr (IDX == 2) {
        src = p.x_rows[s];
      }
      xvo[c] = r < sl.rows
                   ? (static_cast<uint32_t>(src) * static_cast<uint32_t>(Kd) + static_cast<uint32_t>(la * 8)) * 2u
                   : x_bytes;
    }
  };
  set_load_slab(slab(0));

  // The loads of the next stage of the load side into ring slot `slot`; past
  // the wave's last stage the same loads at offsets past the end.
  // (Conditions below combine with & rather than &&: short-circuit forms
  // became branches, each with its own copy of the load.)
  auto issue = [&](int slot) {
    const bool live = li < my;
    const int k0 = lkk * kBK;
    u32x4_t* base = ring(slot);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool ok = live & (wvo[j] < w_bytes) & (k0 + wkc[j] < Kd);
        lds_load16_nt(rw[m], ok ? wvo[j] + k0 * 2 : w_bytes, base + m * kSlabRows * kCH + j * 64);
      }
#pragma unroll
    for (int c = 0; c < MC; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = k0 + u * 32;
        const bool ok = live & (xvo[c] < x_bytes) & (k + la * 8 < Kd);
        lds_load16(rx, ok ? xvo[c] + k * 2 : x_bytes, 0, base + WSLOT + (c * 2 + u) * 64);
      }
    if (live && ++lkk == nks) {
      lkk = 0;
      if (++li < my) set_load_slab(slab(li));
    }
  };

  // Compute side.
  f32x4_t acc[NMAT][MC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < MC; ++c) acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    const u32x4_t* base = ring(slot);
    bf16x8_t wf[NMAT][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) wf[m][u] = as_bf16x8(base[m * kSlabRows * kCH + swz(lb, 4 * u + la)]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < MC; ++c)
          acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              wf[m][u], as_bf16x8(base[WSLOT + (c * 2 + u) * 64 + lane]), acc[m][c], 0, 0, 0);
  };
  // 16x16 accumulator: lane l holds token row c * 16 + l % 16 and weight rows
  // 4 (l / 16) + i, i = 0..3 (four consecutive output columns).
  auto epilogue = [&](const Slab& sl) {
    const int n = sl.n0 + la * 4;
    if (n >= N) return;  // N % 8 == 0: four columns are all in or all out
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int r = c * 16 + lb;
      if (r >= sl.rows) continue;
      const int s = sl.beg + r;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (MODE == G1_SWIGLU || MODE == G1_GELU) {
          v[i] = epilogue_g1(MODE, acc[0][c][i], acc[NMAT - 1][c][i], p.bias, sl.e, N, n + i);
        } else {
          v[i] = acc[0][c][i];
          if (p.bias != nullptr) v[i] += bf16_to_f32(p.bias[static_cast<size_t>(sl.e) * N + n + i]);
        }
      }
      if (MODE == G1_SWIGLU || MODE == G1_GELU) {
        store_global(static_cast<bf16_t*>(p.out) + static_cast<size_t>(s) * N + n,
                     u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      } else if (MODE == G2_OPERM) {
        store_global(static_cast<float*>(p.out) + static_cast<size_t>(s) * N + n, f32x4_t{v[0], v[1], v[2], v[3]});
      } else {
        const int t = p.slot_token[s];
        const float g = p.gate[t];
        store_global(static_cast<bf16_t*>(p.out) + static_cast<size_t>(t) * N + n,
                     u32x2_t{pack_bf16x2(g * v[0], g * v[1]), pack_bf16x2(g * v[2], g * v[3])});
      }
    }
  };

  // Prologue: stages 0 .. NBUF - 2 into slots 0 .. NBUF - 2. (Every loop over
  // ring slots is fully unrolled, so the register ring's index is a constant.)
#pragma unroll
  for (int sl = 0; sl + 1 < NBUF; ++sl) issue(sl);

  Slab cs = slab(0);
  int ci = 0, ckk = 0;
  // Stage t uses slot t % NBUF and loads stage t + NBUF - 1 into slot
  // (t - 1) % NBUF, read by stage t - 1 (whose fragment reads have completed:
  // its MFMAs consumed them).
  for (int t0 = 0; t0 < nstage; t0 += NBUF) {
#pragma unroll
    for (int sl = 0; sl < NBUF; ++sl) {
      if (t0 + sl < nstage) {
        issue((sl + NBUF - 1) % NBUF);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT));
        asm volatile("" ::: "memory");
        compute(sl);
        if (++ckk == nks) {
          epilogue(cs);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < MC; ++c) acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          ckk = 0;
          if (++ci < my) cs = slab(ci);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in LDS after the block ends
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------- launch

// Compute units of the current device (cached per device; 0 if the query fails).
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, int BN, int WM, int WN, int MODE, bool BT = false, bool XT = false, bool PERSIST = false,
          bool TS = false>
hipError_t launch_tile(GemmParams p, int S, hipStream_t st) {
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  p.n_mt = MODE == G_WGRAD ? p.E * ((p.M + BM - 1) / BM) : (S + BM - 1) / BM + min(p.E, S);
  if (TS) p.n_mt += p.E * (p.ks - 1);  // at most one split tail per expert
  const int n_nt = (p.N + BN / NMAT - 1) / (BN / NMAT);
  const size_t total = static_cast<size_t>(n_nt) * p.n_mt;
  size_t grid = (total + 7) / 8 * 8;
  if (PERSIST) {  // one block per CU, a multiple of 8 (every XCD the same count)
    const size_t cus = static_cast<size_t>(device_cu_count()) / 8 * 8;
    if (cus >= 8 && cus < grid) grid = cus;
  }
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, WN, MODE, BT, XT, PERSIST, TS>),
                     dim3(static_cast<unsigned>(grid)), dim3(WM * WN * 64), 0, st, p);
  return hipGetLastError();
}

// 256 x 256 tiles: about 1k rows per expert and at least two tiles per CU.
bool tiles_256(int S, int E, int N, int nmat) {
  const long bn = 256 / nmat;
  const long blocks = static_cast<long>((S + 255) / 256 + min(E, S)) * ((N + bn - 1) / bn);
  return S / max(E, 1) >= 512 && blocks >= 2 * 256;
}

// Split tails of the second GEMM. On 256 x 256 tiles a tail of at most 64 rows
// (the last m-tile of an expert) keeps one of four wave rows busy but streams a
// whole weight slice over the full reduction; at the prefill shape the 64 tail
// tiles beside 512 full ones made a third, mostly idle round (second GEMM
// 0.96 ms against 0.80 ms for the same rows in whole tiles). Split into
// kTailSplit parts along k they run as short tiles among the full ones; part j
// writes float32 partial rows, and tail_sum_kernel adds the parts in order
// 0, 1, ... into o_perm (fixed order: the same bits every run).
constexpr int kTailSplit = 4;
constexpr int kTailRows = 64;  // rows of one wave row of a 256 x 256 tile (4 x 2 waves)

__global__ __launch_bounds__(256) void tail_sum_kernel(const float* __restrict__ part, float* __restrict__ o_perm,
                                                       const int32_t* __restrict__ offsets, int S, int cap, int E,
                                                       int N, int ks) {
  const int e = static_cast<int>(blockIdx.x) / kTailRows, r = static_cast<int>(blockIdx.x) % kTailRows;
  int b, en;
  expert_rows(offsets, e, S, cap, &b, &en);
  const int cnt = en - b, rem = cnt % 256;
  if (rem == 0 || rem > kTailRows || r >= rem) return;
  float* dst = o_perm + static_cast<size_t>(b + cnt - rem + r) * N;
  for (int c = static_cast<int>(threadIdx.x) * 4; c < N; c += 256 * 4) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + (static_cast<size_t>(e) * kTailRows + r) * N + c);
    for (int j = 1; j < ks; ++j) {
      const f32x4_t w = *reinterpret_cast<const f32x4_t*>(
          part + (static_cast<size_t>(j * E + e) * kTailRows + r) * N + c);
      v = f32x4_t{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
    }
    *reinterpret_cast<f32x4_t*>(dst + c) = v;
  }
}

// Tile shape from the mean rows per expert (S / E): with about 1k rows per
// expert, 256 x 256 tiles (the fewest bytes moved per flop) on 8 waves, two per
// SIMD, so that one wave's MFMAs run while the other waits (4 waves of
// 128 x 128, which read a third fewer LDS bytes per MFMA, measured slower on
// every GEMM once the 8-wave kernel raised its priority around the MFMAs and
// the dZ GEMM's epilogue issued its loads ahead of its stores: dZ GEMM
// 1.47 -> 1.37 ms on 8 waves). With about 100
// rows per expert, 128 x 256 tiles on 8 waves with the weights two stages
// ahead (measured on the Switch-style layer: 21 % faster than one stage ahead
// on the first GEMM; on the second 5 % faster than 128 x 128 tiles at two
// blocks per CU). Small grids fall back to 128 x 128 so that the chip is
// still covered.
template <int MODE, bool BT = false>
hipError_t launch_tile_auto(GemmParams p, int S, hipStream_t st) {
  constexpr bool G1 = (MODE == G1_SWIGLU || MODE == G1_GELU || MODE == G1_SWIGLU_Z || MODE == G1_GELU_Z);
  constexpr int NMAT = (MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) ? 2 : 1;
  const int mean_rows = S / max(p.E, 1);
  auto blocks = [&](int bm, int bn) {
    return static_cast<long>((S + bm - 1) / bm + min(p.E, S)) * ((p.N + bn / NMAT - 1) / (bn / NMAT));
  };
  if (mean_rows >= 512 && blocks(256, 256) >= 2 * 256) {
    // persistent tiles where the epilogue reads nothing (measured: prefill first
    // GEMM -2 %, backward recompute -1 %; the second GEMM, 2.25 tiles per CU,
    // +2.5 % with the static tile order)
    if constexpr ((MODE == G1_SWIGLU || MODE == G1_SWIGLU_Z) && !BT) {
      return launch_tile<256, 256, 4, 2, MODE, BT, false, true>(p, S, st);
    } else {
      return launch_tile<256, 256, 4, 2, MODE, BT>(p, S, st);
    }
  }
  if (blocks(128, 256) >= 2 * 256) return launch_tile<128, 256, 4, 2, MODE, BT>(p, S, st);
  return launch_tile<128, 128, 2, 2, MODE, BT>(p, S, st);
}

// Waves of the slab kernel: as many as fit (LDS ring and registers allow
// `per_cu` per CU), but cut so that every wave gets the same number of slabs
// when every expert is hit.
template <int MODE, int MC, int NBUF>
hipError_t launch_slab_mc(GemmParams p, hipStream_t st) {
  constexpr int NMAT = (MODE == G1_SWIGLU) ? 2 : 1;
  constexpr int ring_bytes = NBUF * (NMAT * kSlabRows * kCH + MC * 2 * 64) * 16;
  const int per_cu = std::min(8, 160 * 1024 / ring_bytes);
  const long slabs = static_cast<long>(p.E) * ((p.N + kSlabRows - 1) / kSlabRows);
  const long cap = 256L * per_cu;
  const long per_wave = (slabs + cap - 1) / cap;
  const dim3 grid(static_cast<unsigned>((slabs + per_wave - 1) / per_wave));
  if (p.x_rows == nullptr) {
    hipLaunchKernelGGL((gemm_slab_kernel<MODE, MC, NBUF, 0>), grid, dim3(64), 0, st, p);
  } else if (p.S <= kSlabIdsMax) {
    hipLaunchKernelGGL((gemm_slab_kernel<MODE, MC, NBUF, 1>), grid, dim3(64), 0, st, p);
  } else {
    hipLaunchKernelGGL((gemm_slab_kernel<MODE, MC, NBUF, 2>), grid, dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

template <int MODE, int NBUF>
hipError_t launch_slab(GemmParams p, int max_rows, hipStream_t st) {
  return max_rows <= 16 ? launch_slab_mc<MODE, 1, NBUF>(p, st) : launch_slab_mc<MODE, 2, NBUF>(p, st);
}

constexpr int kSlabMaxRows = 32;  // rows per expert up to which the slab kernel runs

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
  if (f.max_rows_per_expert <= kSlabMaxRows) {
    return swiglu ? launch_slab<G1_SWIGLU, kSlabBuf1>(p, f.max_rows_per_expert, st)
                  : launch_slab<G1_GELU, kSlabBuf1>(p, f.max_rows_per_expert, st);
  }
  return swiglu ? launch_tile_auto<G1_SWIGLU>(p, f.S, st) : launch_tile_auto<G1_GELU>(p, f.S, st);
}

size_t gemm2_tail_bytes(int S, int E, int d, int width, int max_rows_per_expert, bool fused_y) {
  if (fused_y || max_rows_per_expert <= kSlabMaxRows || !tiles_256(S, E, d, 1)) return 0;
  if ((width + 63) / 64 < 4 * kTailSplit) return 0;  // every part at least four stages
  return static_cast<size_t>(kTailSplit) * E * kTailRows * d * 4;
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
  if (f.max_rows_per_expert <= kSlabMaxRows) {
    return f.fused_y ? launch_slab<G2_FUSED_Y, kSlabBuf2>(p, f.max_rows_per_expert, st)
                     : launch_slab<G2_OPERM, kSlabBuf2>(p, f.max_rows_per_expert, st);
  }
  if (f.tail_part != nullptr && gemm2_tail_bytes(f.S, f.E, f.d, f.width, f.max_rows_per_expert, f.fused_y) > 0) {
    p.tail_part = f.tail_part;
    p.ks = kTailSplit;
    const hipError_t err = launch_tile<256, 256, 4, 2, G2_OPERM, false, false, false, true>(p, f.S, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tail_sum_kernel, dim3(static_cast<unsigned>(f.E * kTailRows)), dim3(256), 0, st,
                       static_cast<const float*>(f.tail_part), f.o_perm, f.offsets, f.S, f.cap, f.E, f.d, kTailSplit);
    return hipGetLastError();
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

size_t bwd_dx_tail_bytes(int S, int E, int d, int Kd) {
  if (!tiles_256(S, E, d, 1) || (Kd + 63) / 64 < 4 * kTailSplit) return 0;
  return static_cast<size_t>(kTailSplit) * E * kTailRows * d * 4;
}

hipError_t launch_bwd_dx_bf16(const void* dZ, int S, const int32_t* offsets, int cap, int E, const void* W1,
                              const void* W3, int N, int Kd1, float* out, float* tail_part, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(dZ);
  p.x_nrows = S;
  p.cap = cap;
  p.offsets = offsets;
  p.B = static_cast<const bf16_t*>(W1);
  p.B3 = static_cast<const bf16_t*>(W3);
  p.kb3 = W3 != nullptr ? Kd1 : 0;
  p.out = out;
  p.E = E;
  p.N = N;
  p.Kd = W3 != nullptr ? 2 * Kd1 : Kd1;
  p.S = S;
  // split tails as in the forward's second GEMM (the same 2.25 rounds of 256 x
  // 256 tiles at the prefill shape, over a reduction of 2 width)
  if (tail_part != nullptr && bwd_dx_tail_bytes(S, E, N, p.Kd) > 0) {
    p.tail_part = tail_part;
    p.ks = kTailSplit;
    const hipError_t err = launch_tile<256, 256, 4, 2, G2_OPERM, true, false, false, true>(p, S, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tail_sum_kernel, dim3(static_cast<unsigned>(E * kTailRows)), dim3(256), 0, st,
                       static_cast<const float*>(tail_part), out, offsets, S, cap, E, N, kTailSplit);
    return hipGetLastError();
  }
  return launch_tile_auto<G2_OPERM, true>(p, S, st);
}

hipError_t launch_bwd_dz_bf16(const void* dy, int T, const int32_t* slot_token, int S, const int32_t* offsets,
                              int cap, int E, const void* W2, int N, int Kd, const void* z, int act,
                              const float* rgate, const void* a, float* dgp, void* dZ, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(dy);
  p.x_rows = slot_token;
  p.x_nrows = T;
  p.cap = cap;
  p.offsets = offsets;
  p.B = static_cast<const bf16_t*>(W2);
  p.zin = static_cast<const bf16_t*>(z);
  p.rgate = rgate;
  p.ain = static_cast<const bf16_t*>(a);
  p.dgp = dgp;
  p.out = dZ;
  p.E = E;
  p.N = N;
  p.Kd = Kd;
  p.S = S;
  return act == 1 ? launch_tile_auto<G2_DZ_SWIGLU, true>(p, S, st) : launch_tile_auto<G2_DZ_GELU, true>(p, S, st);
}

hipError_t launch_bwd_wgrad_bf16(const void* X, int M, const void* B, bool b_kmajor, int N, int ldk,
                                 const int32_t* kofs, const int32_t* offsets, int S, int cap, int E, float* out,
                                 float* out2, int split, hipStream_t st) {
  GemmParams p{};
  p.x = static_cast<const bf16_t*>(X);
  p.B = static_cast<const bf16_t*>(B);
  p.kofs = kofs;
  p.offsets = offsets;
  p.S = S;
  p.cap = cap;
  p.M = M;
  p.ldk = ldk;
  p.split = split;
  p.out = out;
  p.out2 = out2;
  p.E = E;
  p.N = N;
  p.Kd = ldk;
  return b_kmajor ? launch_tile<256, 256, 4, 2, G_WGRAD, true, true>(p, 0, st)
                  : launch_tile<256, 256, 4, 2, G_WGRAD, false, true>(p, 0, st);
}

}  // namespace moe

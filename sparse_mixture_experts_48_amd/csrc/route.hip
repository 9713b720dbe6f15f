// Router of the MoE layer: float32 logits, softmax, top-K, gates, and the
// per-block partial statistics behind the expert counts and the aux loss.
//
// Lensa ML explainer "Mixture of Experts":
//   Step 2 (The Router): logits = h . W_r, then a softmax over the experts.
//   Step 3 (Top-k Routing): keep the K largest; gates are a softmax over the
//     chosen logits (Mixtral), or p_i unrenormalised (Switch top-1).
//   Step 4 (Load Balancing): T*K slots counted per expert; aux = E sum f P.
// Arjun Jaggi, "Mixture of Experts in LLMs", section "Switch Transformers":
//   the router runs in float32.
//
// Numeric contract (the pages leave the summation order open; this one is
// fixed so that the expert choice never depends on how the work is split):
// k is cut into groups of four consecutive values, group g belongs to chain
// g mod 4, each chain is an fmaf chain from +0 over its k in ascending order,
// and logit = (c0 + c1) + (c2 + c3), bias added afterwards. Four independent
// chains per logit instead of one quarter the dependent-latency floor of a
// small batch and give a large batch four times the independent fmas.
//
// Three layouts of the same chains:
//  * MFMA (17..64 experts): the chains run on the float32 matrix cores, whose
//    32x32x2 MFMA applies its two k as two correctly rounded fmas in order
//    (route_mfma_kernel); one wave per chain and 32 experts of a 32-token
//    block, chain sums through LDS, then the per-token epilogue.
//  * wide (up to 16 experts, T > 256): a thread owns one chain of TPT tokens x TE
//    experts and walks that chain's k upward; lanes are laid out as [token
//    group][chain][expert lane], so the four chains of a logit sit LE = EP/TE
//    lanes apart (two xor-butterflies form the sums, identical in all four)
//    and the experts of one token sit in LE adjacent lanes, where the
//    per-token max / argmax / sum reductions are xor-butterflies. Keeping one
//    chain per thread leaves the registers for a larger token x expert tile,
//    which sets the LDS bytes read per fma.
//  * narrow (E <= 16, T <= 256): one token per wave, lane = chain * EP + expert.
//    The wave turns its token's h into float32 once per chunk of k (its own
//    LDS row), the block stages W_r chunks in LDS transposed, and each active
//    lane runs one chain reading four h values and four W_r values per step:
//    no conversion in the chain, and many more waves in flight for small
//    batches. Two butterflies over the chain index form the sums.
#include "common.h"
#include "kernels.h"
#include "stats.h"

namespace moe {

namespace {

constexpr int kRouteThreads = 256;

// Wide layout per padded expert count: TE experts and TPT tokens per thread
// (one chain of each), BK k per LDS stage. A token group takes 4 * EP / TE
// lanes; a block holds kRouteThreads / (4 * EP / TE) * TPT tokens. (More
// experts run on the MFMA layout.)
template <int EP> struct WideCfg;
template <> struct WideCfg<8> { static constexpr int TE = 2, TPT = 1, BK = 128; };
template <> struct WideCfg<16> { static constexpr int TE = 4, TPT = 2, BK = 128; };
template <int EP>
constexpr int wide_tb() { return kRouteThreads / (4 * EP / WideCfg<EP>::TE) * WideCfg<EP>::TPT; }

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// 8 consecutive h values of one token as raw bits (bf16: one 16-byte load).
// Raw buffer over `bytes` bytes at `base`: loads at byte offsets >= bytes
// return zeros. The router's loads go through these, with no branch around
// them, so that the compiler's wait counts keep several stages of loads in
// flight (a load behind a branch makes it wait for every load before a use).
// The range is uniform, but where the compiler forms it with a vector
// instruction (a clamp becomes v_med3) the descriptor would sit in vector
// registers and every load through it would loop over the lanes; reading the
// first lane puts it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t route_rsrc(const void* base, uint32_t bytes) {
  bytes = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes)));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load16f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const uint4 v = load16(r, byte_off);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

template <typename Tin> struct HVec;
template <> struct HVec<float> {
  typedef float4 raw[2];
  // 8 values at element offset `off` of the buffer (zeros past its end)
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, raw& x) {
    x[0] = load16f(r, 4 * off);
    x[1] = load16f(r, 4 * off + 16);
  }
  __device__ __forceinline__ static void zero(raw& r) { r[0] = r[1] = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ static void to_f32(const raw& r, float* out) {
    out[0] = r[0].x; out[1] = r[0].y; out[2] = r[0].z; out[3] = r[0].w;
    out[4] = r[1].x; out[5] = r[1].y; out[6] = r[1].z; out[7] = r[1].w;
  }
};
template <> struct HVec<bf16_t> {
  typedef uint4 raw[1];
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, raw& x) {
    x[0] = load16(r, 2 * off);
  }
  __device__ __forceinline__ static void zero(raw& r) { r[0] = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ static void to_f32(const raw& r, float* out) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// What a router block hands on.
struct RouteOut {
  const float* br;
  const float* noise;
  int T, E, K, gate_mode, bias_select;
  int32_t* topk_idx;
  float* topk_gate;
  float* logits_out;
  int32_t* blk_hist;
  float* blk_psum;
  float* blk_z;
};

// Per-token epilogue of the wide layouts. lsum[i][q] is the float32 sum
// (c0 + c1) + (c2 + c3) of token t0 + tg + i * G, expert expert_of(q), held
// alike by the four chain lanes cj of that token group (lanes with cj == 0
// write). Forms the scores, the top-K and its gates, the softmax's column sums
// and lse^2, and the block's histogram (hist_s, cleared before a barrier that
// precedes this call), then writes the block's partials (has a barrier).
template <int EP, int TE, int TPT, int LE, int G, typename ExpertOf>
__device__ __forceinline__ void route_epilogue(const float (&lsum)[TPT][TE], int tg, int cj, int el, int t0,
                                               ExpertOf expert_of, const RouteOut& o, float (*psum_s)[EP],
                                               float* z_s, int* hist_s) {
  const int tid = threadIdx.x;
  const float* br = o.br;
  const float* noise = o.noise;
  const int T = o.T, E = o.E, K = o.K, gate_mode = o.gate_mode, bias_select = o.bias_select;
  int32_t* topk_idx = o.topk_idx;
  float* topk_gate = o.topk_gate;
  float* logits_out = o.logits_out;
  int32_t* blk_hist = o.blk_hist;
  float* blk_psum = o.blk_psum;
  float* blk_z = o.blk_z;
  float psum_local[TE];
#pragma unroll
  for (int q = 0; q < TE; ++q) psum_local[q] = 0.0f;
  float z_local = 0.0f;  // sum of lse^2 over this token group's tokens (z-loss)

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = t0 + tg + i * G;
    const bool tok_ok = t < T;  // uniform across the lanes of this token group
    // l: the score the choice is made on (logit + bias, + noise); lg: the
    // logit of the softmax and the gates (l, or logit + noise when the bias
    // only steers the choice)
    float l[TE], lg[TE];
#pragma unroll
    for (int q = 0; q < TE; ++q) {
      const int e = expert_of(q);
      const float c0123 = lsum[i][q];
      if (e < E) {
        l[q] = c0123;
        if (br != nullptr) l[q] = l[q] + br[e];
        lg[q] = bias_select ? c0123 : l[q];
        if (noise != nullptr && tok_ok) {
          const float nz = noise[static_cast<size_t>(t) * E + e];
          l[q] = l[q] + nz;
          lg[q] = lg[q] + nz;
        }
      } else {
        l[q] = -INFINITY;
        lg[q] = -INFINITY;
      }
    }
    if (tok_ok && cj == 0 && logits_out != nullptr) {
#pragma unroll
      for (int q = 0; q < TE; ++q) {
        const int e = expert_of(q);
        if (e < E) logits_out[static_cast<size_t>(t) * E + e] = l[q];
      }
    }
    // top-K by (logit descending, expert ascending)
    bool taken[TE];
#pragma unroll
    for (int q = 0; q < TE; ++q) taken[q] = false;
    int cidx[8];
    float cval[8], cg[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        float bv = -INFINITY, bg = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < TE; ++q) {
          const int e = expert_of(q);
          if (!taken[q] && e < E && better(l[q], e, bv, bi)) { bv = l[q]; bi = e; bg = lg[q]; }
        }
#pragma unroll
        for (int off = 1; off < LE; off <<= 1) {
          const float ov = __shfl_xor(bv, off, LE);
          const int oi = __shfl_xor(bi, off, LE);
          const float og = __shfl_xor(bg, off, LE);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; bg = og; }
        }
        cidx[j] = bi;
        cval[j] = bv;
        cg[j] = bg;
#pragma unroll
        for (int q = 0; q < TE; ++q)
          if (expert_of(q) == bi) taken[q] = true;
      }
    }
    // softmax over all E (the largest lg is the first choice, unless the
    // bias steers the choice)
    float m = cval[0];
    if (bias_select) {
      m = lg[0];
#pragma unroll
      for (int q = 1; q < TE; ++q) m = fmaxf(m, lg[q]);
#pragma unroll
      for (int off = 1; off < LE; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, LE));
    }
    float ex[TE];
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < TE; ++q) {
      ex[q] = (expert_of(q) < E) ? expf(lg[q] - m) : 0.0f;
      s += ex[q];
    }
#pragma unroll
    for (int off = 1; off < LE; off <<= 1) s += __shfl_xor(s, off, LE);
    if (tok_ok) {
#pragma unroll
      for (int q = 0; q < TE; ++q) psum_local[q] += ex[q] / s;
      const float lse = m + logf(s);
      z_local += lse * lse;
    }
    if (tok_ok && cj == 0 && el == 0) {
      float ec[8];
      float se = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          ec[j] = expf(cg[j] - m);
          se += ec[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          const float g = (gate_mode == 0) ? ec[j] / se : ec[j] / s;
          topk_idx[static_cast<size_t>(t) * K + j] = cidx[j];
          topk_gate[static_cast<size_t>(t) * K + j] = g;
          // a token whose scores are NaN chooses no expert (id 0x7fffffff): not counted
          if (static_cast<unsigned>(cidx[j]) < static_cast<unsigned>(E)) atomicAdd(&hist_s[cidx[j]], 1);
        }
      }
    }
  }

#pragma unroll
  for (int q = 0; q < TE; ++q)
    if (cj == 0) psum_s[tg][expert_of(q)] = psum_local[q];
  if (cj == 0 && el == 0) z_s[tg] = z_local;
  __syncthreads();
  if (tid < E) {
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += psum_s[g][tid];
    blk_psum[static_cast<size_t>(blockIdx.x) * E + tid] = s;
    blk_hist[static_cast<size_t>(blockIdx.x) * E + tid] = hist_s[tid];
  }
  if (tid == 0 && blk_z != nullptr) {
    float z = 0.0f;
    for (int g = 0; g < G; ++g) z += z_s[g];  // fixed order
    blk_z[blockIdx.x] = z;
  }
}

// EP: experts padded to a power of two; TE experts and TPT tokens per thread;
// BK: k values per LDS stage; NS: pipeline depth (NS - 1 stages of global
// loads in flight in registers while one stage is consumed from LDS).
template <typename Tin, int EP, int TE, int TPT, int BK, int NS>
__global__ __launch_bounds__(kRouteThreads) void route_wide_kernel(
    const Tin* __restrict__ h, const float* __restrict__ Wr, const float* __restrict__ br,
    const float* __restrict__ noise, int T, int d, int E, int K, int gate_mode,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, float* __restrict__ logits_out,
    int32_t* __restrict__ blk_hist, float* __restrict__ blk_psum, float* __restrict__ blk_z, int bias_select) {
  constexpr int LE = EP / TE;             // expert lanes per chain
  constexpr int LG = 4 * LE;              // lanes per token group: chain-major, then expert lane
  constexpr int G = kRouteThreads / LG;   // token groups per block
  constexpr int TB = G * TPT;             // tokens per block
  static_assert(LE >= 1 && LG <= 64 && (64 % LG) == 0, "token-group lanes must tile a wave");
  constexpr int HP = BK + 4;              // h_s row stride (floats)
  constexpr int WP = EP + 4;              // w_s row stride (floats)
  constexpr int HN = TB * (BK / 8);                        // 8-value h vectors per stage
  constexpr int HV = (HN + kRouteThreads - 1) / kRouteThreads;  // ... per thread
  constexpr int WV = (BK * EP / 4 + kRouteThreads - 1) / kRouteThreads;  // W_r float4s per thread

  __shared__ __align__(16) float h_s[2][TB][HP];
  __shared__ __align__(16) float w_s[2][BK][WP];
  __shared__ float psum_s[G][EP];
  __shared__ float z_s[G];
  __shared__ int hist_s[EP];

  const int tid = threadIdx.x;
  const int tg = tid / LG;
  const int cj = (tid % LG) / LE;  // chain of this lane
  const int el = tid % LE;
  // Expert q of this lane. With TE a multiple of 4 the lane's experts are
  // float4 runs at el*4, el*4 + 4*LE, ...: the LE lanes of one read then touch
  // consecutive 16-byte slots of a w_s row (no bank conflicts).
  auto expert_of = [&](int q) { return TE % 4 == 0 ? (q / 4) * (4 * LE) + el * 4 + q % 4 : el * TE + q; };
  const int t0 = blockIdx.x * TB;
  if (tid < EP) hist_s[tid] = 0;
  const int nc = (d + BK - 1) / BK;

  typename HVec<Tin>::raw hreg[NS][HV];
  float4 wreg[NS][WV];

  // The block's token rows (rows past T read zeros) and all of W_r as buffers.
  const int rows = max(0, min(TB, T - t0));
  const __amdgpu_buffer_rsrc_t hbuf =
      route_rsrc(h + static_cast<size_t>(min(t0, max(T - 1, 0))) * d, static_cast<uint32_t>(rows) * d * sizeof(Tin));
  const __amdgpu_buffer_rsrc_t wbuf = route_rsrc(Wr, static_cast<uint32_t>(d) * E * 4);
  // Issue the global loads of stage c into register slot `slot`. Stages past
  // the end are allowed (zeros or values that are never stored). In the last
  // stage, h values at k >= d of a row come from the next row: never read
  // (the chains stop at d) — rows past the block's last one read zeros.
  auto load_stage = [&](int c, int slot) {
    const int k0 = c * BK;
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kRouteThreads;
      const int r = i / (BK / 8);
      const int cc = (i % (BK / 8)) * 8;
      HVec<Tin>::load(hbuf, static_cast<uint32_t>(r) * d + k0 + cc, hreg[slot][v]);
    }
    // rows k0 .. of W_r are one contiguous run of floats; values past the
    // stage's run are never stored, values past W_r are zeros
#pragma unroll
    for (int v = 0; v < WV; ++v) {
      const int i = tid + v * kRouteThreads;
      wreg[slot][v] = load16f(wbuf, (static_cast<uint32_t>(k0) * E + 4 * i) * 4);
    }
  };
  // Padded experts read zeros; no stage writes their columns, so both buffers
  // are cleared once (the first stage's barrier orders this before any read).
  if (E < EP) {
    const int pad = EP - E;
    for (int i = tid; i < 2 * BK * pad; i += kRouteThreads) {
      const int b = i / (BK * pad);
      const int r = i - b * (BK * pad);
      w_s[b][r / pad][E + r % pad] = 0.0f;
    }
  }
  // Row of element f of a stage's W_r run: f / E as (f * ceil(2^32 / E)) >> 32,
  // exact for f < 2^16 (a stage holds at most BK * E <= 8192 floats).
  const uint64_t e_recip = (0x100000000ull + E - 1) / E;
  // Move register slot `slot` (stage c) into LDS buffer `buf`.
  auto store_stage = [&](int c, int slot, int buf) {
    const int kn = min(BK, d - c * BK);
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kRouteThreads;
      const int r = i / (BK / 8);
      const int cc = (i % (BK / 8)) * 8;
      if (HN % kRouteThreads != 0 && i >= HN) continue;
      float x[8];
      HVec<Tin>::to_f32(hreg[slot][v], x);
      *reinterpret_cast<float4*>(&h_s[buf][r][cc]) = make_float4(x[0], x[1], x[2], x[3]);  // HP % 4 == 0
      *reinterpret_cast<float4*>(&h_s[buf][r][cc + 4]) = make_float4(x[4], x[5], x[6], x[7]);
    }
    const int n4 = kn * E / 4;
#pragma unroll
    for (int v = 0; v < WV; ++v) {
      const int i = tid + v * kRouteThreads;
      if (i < n4) {
        int k = static_cast<int>((static_cast<uint64_t>(4 * i) * e_recip) >> 32);
        int e = 4 * i - k * E;
        if (E % 4 == 0) {  // the four floats sit in one row: one 16-byte store (WP % 4 == 0)
          *reinterpret_cast<float4*>(&w_s[buf][k][e]) = wreg[slot][v];
        } else {
          const float x[4] = {wreg[slot][v].x, wreg[slot][v].y, wreg[slot][v].z, wreg[slot][v].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            w_s[buf][k][e] = x[u];
            if (++e == E) { e = 0; ++k; }
          }
        }
      }
    }
  };

  float acc[TPT][TE];  // chain cj of each of the thread's logits
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int q = 0; q < TE; ++q) acc[i][q] = 0.0f;

  // One group of four k (kk .. kk+3 of the stage) for this lane's chain.
  auto compute_group = [&](int buf, int kk) {
    float4 hv[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) hv[i] = *reinterpret_cast<const float4*>(&h_s[buf][tg + i * G][kk]);
    float wv[4][TE];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (TE % 4 == 0) {
#pragma unroll
        for (int q4 = 0; q4 < TE; q4 += 4) {
          const float4 w4 = *reinterpret_cast<const float4*>(&w_s[buf][kk + s][expert_of(q4)]);
          wv[s][q4] = w4.x; wv[s][q4 + 1] = w4.y; wv[s][q4 + 2] = w4.z; wv[s][q4 + 3] = w4.w;
        }
      } else if constexpr (TE == 2) {
        const float2 w2 = *reinterpret_cast<const float2*>(&w_s[buf][kk + s][el * TE]);
        wv[s][0] = w2.x; wv[s][1] = w2.y;
      } else {
#pragma unroll
        for (int q = 0; q < TE; ++q) wv[s][q] = w_s[buf][kk + s][el * TE + q];
      }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const float hk[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q = 0; q < TE; ++q) acc[i][q] = fmaf(hk[s], wv[s][q], acc[i][q]);
    }
  };
  // Chain cj takes the groups 4m + cj of the stage (BK is a multiple of 16, so
  // the stage offset does not move the round-robin), in ascending k.
  static_assert(BK % 16 == 0, "a stage holds whole rounds of the four chains");
  auto compute_stage = [&](int c, int buf) {
    const int ng = min(BK, d - c * BK) / 4;  // groups in the stage (kn is a multiple of 8)
    if (ng == BK / 4) {
      // fully unrolled so that LDS reads run ahead of the fmas
#pragma unroll
      for (int m = 0; m < BK / 16; ++m) compute_group(buf, 16 * m + 4 * cj);
    } else {
      for (int m = 0; 4 * m + cj < ng; ++m) compute_group(buf, 16 * m + 4 * cj);
    }
  };

  // Pipeline: stage c is loaded into register slot c % NS, NS-1 stages before
  // it is stored to LDS buffer c % 2 and consumed; one barrier per stage. The
  // main loop issues its loads with no condition (past the end they are
  // unused); the tail, fewer than NS stages, has all of its stages loaded.
  static_assert(NS % 2 == 0, "slot parity selects the LDS buffer");
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) load_stage(s, s);
  int c0 = 0;
  for (; c0 + NS <= nc; c0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      store_stage(c0 + s, s, s & 1);
      __syncthreads();
      load_stage(c0 + s + NS - 1, (s + NS - 1) % NS);
      compute_stage(c0 + s, s & 1);
    }
  }
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if (c0 + s < nc) {
      store_stage(c0 + s, s, s & 1);
      __syncthreads();
      compute_stage(c0 + s, s & 1);
    }
  }

  // (c0 + c1) + (c2 + c3): every chain's lane ends with the same sums
  float lsum[TPT][TE];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int q = 0; q < TE; ++q) {
      const float c01 = acc[i][q] + __shfl_xor(acc[i][q], LE);
      lsum[i][q] = c01 + __shfl_xor(c01, 2 * LE);
    }
  const RouteOut o{br, noise, T, E, K, gate_mode, bias_select, topk_idx, topk_gate, logits_out,
                   blk_hist, blk_psum, blk_z};
  route_epilogue<EP, TE, TPT, LE, G>(lsum, tg, cj, el, t0, expert_of, o, psum_s, z_s, hist_s);
}

// MFMA layout (17..64 experts): the four chains on the float32 matrix cores.
// v_mfma_f32_32x32x2_f32 adds to each of its 32 x 32 outputs the products of
// its two k in order, each with one rounding: an fmaf for the first k, then
// one for the second (checked on the hardware against correctly rounded fmaf
// chains, bit for bit, with denormals, infinities, NaN and signed zeros). So
// chain j of a logit is a run of these MFMAs over its k pairs in ascending
// order from a zero accumulator: the same bits as the fmaf chain.
// A block holds 32 tokens; wave w runs chain w % 4 for experts 32 (w / 4) ..
// + 31 with one 32 x 32 accumulator (16 registers). Per 16 k (one group of four
// k per chain) a wave issues two MFMAs: k 4j, 4j+1 and k 4j+2, 4j+3. MFMA
// operands: lane l gives A[token l % 32][k0 + l / 32] and B[k0 + l / 32][expert
// l % 32]. Stages of 64 k of h and W_r go to LDS by direct loads, kMfmaRing - 1
// stages ahead; h rows are stored in 16 units of four k per row, unit c of
// token r at c ^ (r & 15), so the 32 tokens of a read fall in distinct banks
// pairwise. The four chains meet in LDS as (c0 + c1) + (c2 + c3) and go to the
// wide layout's per-token epilogue.
constexpr int kMfmaBK = 64;   // k per stage
constexpr int kMfmaRing = 3;  // register ring: stages loaded ahead of their store to LDS
constexpr int kMfmaTB = 32;   // tokens per block

template <int EP> constexpr int mfma_threads() { return EP / 32 * 4 * 64; }

template <typename Tin, int EP>
__global__ __launch_bounds__(mfma_threads<EP>()) void route_mfma_kernel(
    const Tin* __restrict__ h, const float* __restrict__ Wr, const float* __restrict__ br,
    const float* __restrict__ noise, int T, int d, int E, int K, int gate_mode,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, float* __restrict__ logits_out,
    int32_t* __restrict__ blk_hist, float* __restrict__ blk_psum, float* __restrict__ blk_z, int bias_select) {
  constexpr int NT = mfma_threads<EP>();
  constexpr int TB = kMfmaTB;
  constexpr int S = static_cast<int>(sizeof(Tin));
  constexpr int UG = 4 * S;                  // bytes of one unit: four k of one token
  constexpr int HROW = kMfmaBK * S;          // bytes of one token's stage (16 units)
  constexpr int HB = TB * HROW;              // h bytes per stage
  constexpr int WF = kMfmaBK * EP;           // W_r floats per stage ([64 k][EP])
  constexpr int HP = HB / (NT * 8);          // 8-byte h pieces per thread per stage
  constexpr int WL = WF / (NT * 4);          // float4 W_r pieces per thread per stage
  constexpr int RD = kMfmaRing;              // register ring: stages loaded ahead
  static_assert(HP * NT * 8 == HB && WL * NT * 4 == WF, "whole pieces per thread");
  // epilogue: one token per group of LE lanes, four experts per lane (the
  // chain sums are already formed, so no chain replicas)
  constexpr int TE = 4, LE = EP / TE, G = NT / LE, TPT = TB / G;
  static_assert(G * TPT == TB && TPT == 1, "the epilogue covers the block's tokens, one per lane group");
  constexpr int CP = EP + 4;                 // chain-sum row stride (floats)

  // Three LDS slots: the stage whose operands are read (one stage before its
  // MFMAs), the next one, and the one being stored from the register ring.
  // h rows: unit c of token r at c ^ (r & 15).
  __shared__ __align__(16) char hs[3][HB];
  __shared__ __align__(16) float ws[3][WF];
  __shared__ __align__(16) float cs[4][TB][CP];
  __shared__ float psum_s[G][EP];
  __shared__ float z_s[G];
  __shared__ int hist_s[EP];
  auto hslot = [&](int b) { return &hs[b][0]; };
  auto wslot = [&](int b) { return &ws[b][0]; };

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int j = wid % 4, eh = wid / 4;  // chain, expert half
  const int q = lane / 32, li = lane % 32;
  const int t0 = blockIdx.x * TB;
  if (tid < EP) hist_s[tid] = 0;

  // The block's token rows (rows past T read zeros) and all of W_r as buffers;
  // a stage's offset is the scalar operand, which the range check includes.
  const int rows = max(0, min(TB, T - t0));
  const __amdgpu_buffer_rsrc_t hbuf =
      route_rsrc(h + static_cast<size_t>(min(t0, max(T - 1, 0))) * d, static_cast<uint32_t>(rows) * d * S);
  const __amdgpu_buffer_rsrc_t wbuf = route_rsrc(Wr, static_cast<uint32_t>(d) * E * 4);
  // Per thread: global byte offsets at stage 0 and LDS byte offsets of its
  // pieces. h: consecutive threads take consecutive 8 bytes of a row (whole
  // lines); W_r: float4 f of the stage's [64 k][EP] tile is W_r[k0 + f / EP]
  // [f % EP] (experts past E land in padded columns that are never used).
  uint32_t hvo[HP], hlo[HP], wvo[WL];
#pragma unroll
  for (int p = 0; p < HP; ++p) {
    const int n = tid + p * NT;
    const int r = n / (HROW / 8), lb = (n % (HROW / 8)) * 8;
    hvo[p] = static_cast<uint32_t>(r) * d * S + lb;
    hlo[p] = r * HROW + (((lb / UG) ^ (r & 15)) * UG) + lb % UG;
  }
#pragma unroll
  for (int u = 0; u < WL; ++u) {
    const int f = 4 * (tid + u * NT);
    wvo[u] = (static_cast<uint32_t>(f / EP) * E + f % EP) * 4;
  }
  uint2 hreg[RD][HP];
  float4 wreg[RD][WL];
  // Stage st into register slot rs (a constant: the loops over slots are
  // unrolled). Stages past the end read zeros or values that are never used.
  auto load_stage = [&](int st, int rs) {
#pragma unroll
    for (int p = 0; p < HP; ++p) {
      typedef unsigned int u2 __attribute__((ext_vector_type(2)));
      const u2 v = __builtin_amdgcn_raw_buffer_load_b64(hbuf, static_cast<int>(hvo[p]), st * kMfmaBK * S, 0);
      hreg[rs][p] = make_uint2(v.x, v.y);
    }
#pragma unroll
    for (int u = 0; u < WL; ++u) {
      typedef unsigned int u4 __attribute__((ext_vector_type(4)));
      const u4 v = __builtin_amdgcn_raw_buffer_load_b128(wbuf, static_cast<int>(wvo[u]), st * kMfmaBK * E * 4, 0);
      wreg[rs][u] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
  };
  auto store_stage = [&](int rs, int b) {
#pragma unroll
    for (int p = 0; p < HP; ++p) *reinterpret_cast<uint2*>(hslot(b) + hlo[p]) = hreg[rs][p];
#pragma unroll
    for (int u = 0; u < WL; ++u) *reinterpret_cast<float4*>(wslot(b) + 4 * (tid + u * NT)) = wreg[rs][u];
  };

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  // MFMAs of stage st (ring slot b): rounds of 16 k; chain j's group of four
  // k of a round exists when it starts before d (d is a multiple of 8).
  // Operands of one stage for this wave: per round of 16 k, the A values of
  // k 4j + q and 4j + 2 + q (lane q = l / 32) and the matching B values.
  struct Ops {
    float a0[4], a1[4], b0[4], b1[4];
  };
  Ops ops[2];
  auto read_ops = [&](int b, Ops& o) {
    const char* hrow = hslot(b) + li * HROW;
#pragma unroll
    for (int mm = 0; mm < kMfmaBK / 16; ++mm) {
      const int unit = (4 * mm + j) ^ (li & 15);
      if constexpr (S == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(hrow + unit * UG);
        o.a0[mm] = __uint_as_float(q ? (v.x & 0xFFFF0000u) : (v.x << 16));
        o.a1[mm] = __uint_as_float(q ? (v.y & 0xFFFF0000u) : (v.y << 16));
      } else {
        const float4 v = *reinterpret_cast<const float4*>(hrow + unit * UG);
        o.a0[mm] = q ? v.y : v.x;
        o.a1[mm] = q ? v.w : v.z;
      }
      const float* wrow = wslot(b) + (16 * mm + 4 * j + q) * EP + 32 * eh + li;
      o.b0[mm] = wrow[0];
      o.b1[mm] = wrow[2 * EP];
    }
  };
  // MFMAs of stage st: chain j's group of four k of a round exists when it
  // starts before d (d is a multiple of 8).
  auto mfmas = [&](auto full, int st, const Ops& o) {
    const int kv = d - st * kMfmaBK;
#pragma unroll
    for (int mm = 0; mm < kMfmaBK / 16; ++mm) {
      if (decltype(full)::value || 16 * mm + 4 * j < kv) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(o.a0[mm], o.b0[mm], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(o.a1[mm], o.b1[mm], acc, 0, 0, 0);
      }
    }
  };

  // Stage x lives in register slot x % RD from its load until its store, then
  // in LDS slot x % 3. Each stage st: a barrier (every wave is done with the
  // reads of stage st - 1, made during stage st - 2, so its LDS slot may be
  // overwritten, and the stores of stage st + 1 are visible), the store of
  // stage st + 2 from its registers, the loads of stage st + 2 + RD into the
  // registers just freed, then the operand reads of stage st + 1 and the MFMAs
  // of stage st (whose operands were read during stage st - 1), which the
  // reads overlap. Loads run RD + 2 stages ahead of their MFMAs. The main loop
  // runs whole groups of U full stages with no condition; the tail, at most U
  // stages, has the conditions.
  constexpr int U = RD * 2;  // a multiple of RD, 3 and 2 (RD = 3)
  static_assert(RD == 3, "unroll factor");
  auto stage = [&](auto full, int st, int r) {
    __syncthreads();
    store_stage((r + 2) % RD, (r + 2) % 3);
    load_stage(st + 2 + RD, (r + 2) % RD);
    // keep the loads here: sunk to the end of the stage, the next stage's
    // stores would wait for them
    __builtin_amdgcn_sched_barrier(0);
    read_ops((r + 1) % 3, ops[(r + 1) % 2]);
    mfmas(full, st, ops[r % 2]);
  };
  const int nst = (d + kMfmaBK - 1) / kMfmaBK;  // stages
  const int nfull = d / kMfmaBK;                // stages of a whole 64 k
#pragma unroll
  for (int r = 0; r < RD; ++r) load_stage(r, r);
  store_stage(0, 0);
  store_stage(1, 1);
  load_stage(RD, 0);
  load_stage(RD + 1, 1);
  __syncthreads();
  read_ops(0, ops[0]);
  int s0 = 0;
  for (; s0 + U <= nfull; s0 += U) {
#pragma unroll
    for (int r = 0; r < U; ++r) stage(std::true_type{}, s0 + r, r);
  }
#pragma unroll
  for (int r = 0; r < U; ++r)
    if (s0 + r < nst) stage(std::false_type{}, s0 + r, r);
  // chain sums: accumulator register rg holds token 8 (rg / 4) + 4 q + rg % 4
#pragma unroll
  for (int rg = 0; rg < 16; ++rg) cs[j][8 * (rg / 4) + 4 * q + rg % 4][32 * eh + li] = acc[rg];
  __syncthreads();
  const int tg = tid / LE;
  const int cj = 0;
  const int el = tid % LE;
  auto expert_of = [&](int qq) { return el * 4 + qq; };
  float lsum[TPT][TE];
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int row = tg + u * G;
    const float4 c0 = *reinterpret_cast<const float4*>(&cs[0][row][el * 4]);
    const float4 c1 = *reinterpret_cast<const float4*>(&cs[1][row][el * 4]);
    const float4 c2 = *reinterpret_cast<const float4*>(&cs[2][row][el * 4]);
    const float4 c3 = *reinterpret_cast<const float4*>(&cs[3][row][el * 4]);
    lsum[u][0] = (c0.x + c1.x) + (c2.x + c3.x);
    lsum[u][1] = (c0.y + c1.y) + (c2.y + c3.y);
    lsum[u][2] = (c0.z + c1.z) + (c2.z + c3.z);
    lsum[u][3] = (c0.w + c1.w) + (c2.w + c3.w);
  }
  const RouteOut o{br, noise, T, E, K, gate_mode, bias_select, topk_idx, topk_gate, logits_out,
                   blk_hist, blk_psum, blk_z};
  route_epilogue<EP, TE, TPT, LE, G>(lsum, tg, cj, el, t0, expert_of, o, psum_s, z_s, hist_s);
}

// Narrow layout: kNarrowNW waves per block, one token per wave; chunks of kNarrowKC k,
// the global loads of kNarrowPD chunks in flight. (A deeper ring measured no
// faster: a chunk's fmaf chains, not its loads, set the pace.)
constexpr int kNarrowKC = 512;
constexpr int kNarrowNW = 4;
constexpr int kNarrowPD = 2;

template <typename Tin, int EP, int NW>
__global__ __launch_bounds__(NW * 64) void route_narrow_kernel(
    const Tin* __restrict__ h, const float* __restrict__ Wr, const float* __restrict__ br,
    const float* __restrict__ noise, int T, int d, int E, int K, int gate_mode,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, float* __restrict__ logits_out,
    int32_t* __restrict__ blk_hist, float* __restrict__ blk_psum, float* __restrict__ blk_z, int bias_select) {
  constexpr int KC = kNarrowKC;
  constexpr int NT = NW * 64;
  constexpr int WF4 = KC * EP / 4;         // float4 slots of a W_r chunk buffer
  constexpr int WI = (WF4 + NT - 1) / NT;  // W_r float4 loads per thread per chunk
  static_assert(KC == 8 * 64, "one 8-value h vector per lane per chunk");
  // Separate arrays per buffer, so that reads of one chunk are known not to
  // alias the writes of the next.
  constexpr int RD = 4;                     // ring depth of a chain (steps of one group of 4 k)
  constexpr int HP = KC + 16 * RD;          // h row stride: the ring may read RD rounds past the chunk
  __shared__ __align__(16) float hA[NW][HP];
  __shared__ __align__(16) float hB[NW][HP];
  constexpr int KP = KC + 16 * RD + 4;      // row stride of the transposed chunk (floats)
  __shared__ __align__(16) float wA[EP * KP];  // W_r chunk transposed: [e][k - k0]
  __shared__ __align__(16) float wB[EP * KP];
  __shared__ float psum_s[NW][EP];
  __shared__ float z_s[NW];
  __shared__ int hist_s[EP];

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  if (tid < EP) hist_s[tid] = 0;
  const int t = blockIdx.x * NW + wave;
  const bool tok_ok = t < T;                                 // wave-uniform
  const Tin* hrow = h + static_cast<size_t>(min(t, T - 1)) * d;  // rows past T are dropped
  const __amdgpu_buffer_rsrc_t hbuf = route_rsrc(hrow, static_cast<uint32_t>(d) * sizeof(Tin));
  const __amdgpu_buffer_rsrc_t wbuf = route_rsrc(Wr, static_cast<uint32_t>(d) * E * 4);
  const int nc = (d + KC - 1) / KC;

  constexpr int PD = kNarrowPD;  // register ring of chunks in flight; even, so chunk c uses LDS buffer c % 2
  static_assert(PD % 2 == 0, "ring slot parity selects the LDS buffer");
  typename HVec<Tin>::raw hreg[PD];
  float4 wreg[PD][WI];
  // Register slot `slot` <- chunk c: this lane's 8 h values (zeros past d),
  // and the block's share of W_r (rows k0.. are one run of floats; values past
  // the chunk's run are never stored, values past W_r are zeros). Chunks past
  // the end are allowed.
  auto load_chunk = [&](int c, int slot) {
    const int k0 = c * KC;
    HVec<Tin>::load(hbuf, k0 + 8 * lane, hreg[slot]);
#pragma unroll
    for (int v = 0; v < WI; ++v) {
      const int i = tid + v * NT;
      wreg[slot][v] = load16f(wbuf, (static_cast<uint32_t>(k0) * E + 4 * i) * 4);
    }
  };
  // LDS <- registers: h as float32 in this wave's row; W_r transposed into the
  // block's buffer (element f of the chunk run is row f / E, expert f % E; the
  // quotient is (f * ceil(2^32 / E)) >> 32 in 64 bits, exact for f < 2^16).
  const uint64_t e_recip = (0x100000000ull + E - 1) / E;
  auto store_chunk = [&](int slot, float (*hs)[HP], float* ws) {
    float x[8];
    HVec<Tin>::to_f32(hreg[slot], x);
    *reinterpret_cast<float4*>(&hs[wave][8 * lane]) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(&hs[wave][8 * lane + 4]) = make_float4(x[4], x[5], x[6], x[7]);
#pragma unroll
    for (int v = 0; v < WI; ++v) {
      const int i = tid + v * NT;
      if (i < WF4) {
        const float q[4] = {wreg[slot][v].x, wreg[slot][v].y, wreg[slot][v].z, wreg[slot][v].w};
        int k = static_cast<int>((static_cast<uint64_t>(4 * i) * e_recip) >> 32);
        int e = 4 * i - k * E;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (k < KC) ws[e * KP + k] = q[u];
          if (++e == E) { e = 0; ++k; }
        }
      }
    }
  };

  float acc = 0.0f;
  // Lane (j, e) = (lane / EP, lane % EP) runs chain j of expert e: the groups
  // of four k whose index within the chunk is j mod 4 (KC is a multiple of 16,
  // so chunk boundaries keep the round-robin). One step reads one group of h
  // (the j-lanes of a token read the same address) and of its W_r row into a
  // register ring filled RD steps ahead of the fmas. Both LDS buffers hold
  // zeros past the end of the reduction (h loads past d are zeroed; W_r slots
  // past the run are written with the zeros loaded for them), so a chain runs
  // to a whole number of rings: the extra steps add exact zeros (a chain
  // starts at +0 and a round-to-nearest sum is never -0 unless both terms are).
  const int cj = lane / EP;
  const int ce = lane % EP;
  auto compute = [&](int c, const float (*hs)[HP], const float* ws) {
    if (cj >= 4 || ce >= E) return;
    constexpr int D = RD;
    static_assert(KC % (16 * D) == 0, "ring");
    const int kn = min(KC, d - c * KC);
    const int steps = (kn + 16 * D - 1) / (16 * D) * D;  // rounds of 4 groups, whole rings
    const float4* hw = reinterpret_cast<const float4*>(hs[wave]) + cj;       // HP % 4 == 0
    const float4* wc = reinterpret_cast<const float4*>(ws + ce * KP) + cj;   // KP % 4 == 0
    float4 rh[D], rw[D];
    auto fetch = [&](int slot, int m) {  // reads up to D rounds past `steps` land in the row padding, unused
      rh[slot] = hw[4 * m];
      rw[slot] = wc[4 * m];
    };
    // The ring is filled in slot order (pinned, as the refills below): the
    // wait at the top of the loop then only needs the oldest reads, on entry
    // as on every later pass.
#pragma unroll
    for (int u = 0; u < D; ++u) {
      fetch(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int m = 0; m < steps; m += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        acc = fmaf(rh[u].x, rw[u].x, acc);
        acc = fmaf(rh[u].y, rw[u].y, acc);
        acc = fmaf(rh[u].z, rw[u].z, acc);
        acc = fmaf(rh[u].w, rw[u].w, acc);
        fetch(u, m + u + D);
        // keep the refill here: left to itself the compiler moves every read of
        // the ring to the top of the loop and waits for them, so no read would
        // be in flight while the fmas run
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Chunk c sits in register slot c % PD and LDS buffer c % 2 (A even, B odd).
  // Storing chunk c into a buffer is safe: every wave passed the barrier of
  // chunk c - 1 only after computing chunk c - 2 from that buffer.
  // The main loop issues its loads with no condition (past the end they are
  // unused); the tail, fewer than PD chunks, has all of its chunks loaded.
#pragma unroll
  for (int s = 0; s < PD; ++s) load_chunk(s, s);
  int c0 = 0;
  for (; c0 + PD <= nc; c0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      if (s % 2 == 0) store_chunk(s, hA, wA);
      else store_chunk(s, hB, wB);
      __syncthreads();
      load_chunk(c0 + s + PD, s);
      if (s % 2 == 0) compute(c0 + s, hA, wA);
      else compute(c0 + s, hB, wB);
    }
  }
#pragma unroll
  for (int s = 0; s < PD - 1; ++s) {
    if (c0 + s < nc) {
      if (s % 2 == 0) store_chunk(s, hA, wA);
      else store_chunk(s, hB, wB);
      __syncthreads();
      if (s % 2 == 0) compute(c0 + s, hA, wA);
      else compute(c0 + s, hB, wB);
    }
  }

  // logit = (c0 + c1) + (c2 + c3) on the lanes of chain 0 (lane = expert);
  // lanes of inactive chains or experts hold +0 and are not used
  float part = acc + __shfl_xor(acc, EP);  // chains 0/1: c0 + c1; chains 2/3: c2 + c3
  part = part + __shfl_xor(part, 2 * EP);
  // top-K by (score descending, expert ascending) on l = logit (+ bias)
  // (+ noise); softmax and gates on lg, which is l, or logit + noise when the
  // bias only steers the choice
  float l = -INFINITY;
  float lg = -INFINITY;
  if (lane < E) {
    l = part;
    if (br != nullptr) l = l + br[lane];
    lg = bias_select ? part : l;
    if (noise != nullptr && tok_ok) {
      const float nz = noise[static_cast<size_t>(t) * E + lane];
      l = l + nz;
      lg = lg + nz;
    }
  }
  if (tok_ok && logits_out != nullptr && lane < E) logits_out[static_cast<size_t>(t) * E + lane] = l;
  bool taken = false;
  int cidx[8];
  float cval[8], cg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < K) {
      // a lane is a candidate if its score beats the empty choice (-inf, no
      // expert): any score but NaN, as in the wide layout
      const bool cand = !taken && lane < E && better(l, lane, -INFINITY, 0x7fffffff);
      float bv = cand ? l : -INFINITY;
      int bi = cand ? lane : 0x7fffffff;
      float bg = cand ? lg : -INFINITY;
#pragma unroll
      for (int off = 1; off < EP; off <<= 1) {
        const float ov = __shfl_xor(bv, off, EP);
        const int oi = __shfl_xor(bi, off, EP);
        const float og = __shfl_xor(bg, off, EP);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; bg = og; }
      }
      cidx[j] = bi;
      cval[j] = bv;
      cg[j] = bg;
      if (lane == bi) taken = true;
    }
  }
  float m = cval[0];  // the largest lg: the first choice, unless the bias steers the choice
  if (bias_select) {
    m = lg;
#pragma unroll
    for (int off = 1; off < EP; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, EP));
  }
  const float ex = (lane < E) ? expf(lg - m) : 0.0f;
  float s = ex;
#pragma unroll
  for (int off = 1; off < EP; off <<= 1) s += __shfl_xor(s, off, EP);
  if (lane < EP) psum_s[wave][lane] = tok_ok ? ex / s : 0.0f;
  if (lane == 0) {
    const float lse = m + logf(s);
    z_s[wave] = tok_ok ? lse * lse : 0.0f;
  }
  if (tok_ok && lane == 0) {
    float ec[8];
    float se = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        ec[j] = expf(cg[j] - m);
        se += ec[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        const float g = (gate_mode == 0) ? ec[j] / se : ec[j] / s;
        topk_idx[static_cast<size_t>(t) * K + j] = cidx[j];
        topk_gate[static_cast<size_t>(t) * K + j] = g;
        // a token whose scores are NaN chooses no expert (id 0x7fffffff): not counted
        if (static_cast<unsigned>(cidx[j]) < static_cast<unsigned>(E)) atomicAdd(&hist_s[cidx[j]], 1);
      }
    }
  }
  __syncthreads();
  if (tid < E) {
    float sum = 0.0f;
    for (int w = 0; w < NW; ++w) sum += psum_s[w][tid];  // fixed order
    blk_psum[static_cast<size_t>(blockIdx.x) * E + tid] = sum;
    blk_hist[static_cast<size_t>(blockIdx.x) * E + tid] = hist_s[tid];
  }
  if (tid == 0 && blk_z != nullptr) {
    float z = 0.0f;
    for (int w = 0; w < NW; ++w) z += z_s[w];  // fixed order
    blk_z[blockIdx.x] = z;
  }
}

// Per-block expert histogram of topk_idx, with the router's token tiling.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ topk_idx, int T, int E,
                                                   int K, int TB, int32_t* __restrict__ blk_hist) {
  __shared__ int hist_s[64];
  if (threadIdx.x < 64) hist_s[threadIdx.x] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * TB;
  const int t1 = min(T, t0 + TB);
  for (int v = t0 * K + threadIdx.x; v < t1 * K; v += blockDim.x) {
    const int e = topk_idx[v];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist_s[e], 1);  // ignore invalid ids
  }
  __syncthreads();
  if (threadIdx.x < E) blk_hist[static_cast<size_t>(blockIdx.x) * E + threadIdx.x] = hist_s[threadIdx.x];
}

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const int32_t* __restrict__ blk_hist, const float* __restrict__ blk_psum, const float* __restrict__ blk_z,
    int NB, int T, int E, int K, int32_t* __restrict__ blk_base, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, float* __restrict__ prob_mean, float* __restrict__ aux_out,
    float* __restrict__ z_out) {
  __shared__ int off_s[65];
  finalize_block(blk_hist, blk_psum, blk_z, NB, T, E, K, blk_base, counts_out, offsets_out, prob_mean, aux_out,
                 z_out, off_s);
}

__global__ void zero_outputs_kernel(int E, int32_t* counts, int32_t* offsets, float* prob_mean,
                                    float* aux, float* z_loss) {
  const int i = threadIdx.x;
  if (counts != nullptr && i < E) counts[i] = 0;
  if (prob_mean != nullptr && i < E) prob_mean[i] = 0.0f;
  if (offsets != nullptr && i <= E) offsets[i] = 0;
  if (aux != nullptr && i == 0) *aux = 0.0f;
  if (z_loss != nullptr && i == 0) *z_loss = 0.0f;
}

template <typename Tin, int EP, int TE, int TPT, int BK, int NS>
hipError_t launch_route_wide(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  hipLaunchKernelGGL((route_wide_kernel<Tin, EP, TE, TPT, BK, NS>), dim3(rt.NB), dim3(kRouteThreads), 0, st,
                     static_cast<const Tin*>(a.h), a.Wr, a.br, a.noise, a.T, a.d, a.E, a.K, a.gate, a.topk_idx,
                     a.topk_gate, a.logits, a.blk_hist, a.blk_psum, a.blk_z, a.bias_select);
  return hipGetLastError();
}

template <typename Tin, int EP>
hipError_t launch_route_mfma(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  hipLaunchKernelGGL((route_mfma_kernel<Tin, EP>), dim3(rt.NB), dim3(mfma_threads<EP>()), 0, st,
                     static_cast<const Tin*>(a.h), a.Wr, a.br, a.noise, a.T, a.d, a.E, a.K, a.gate, a.topk_idx,
                     a.topk_gate, a.logits, a.blk_hist, a.blk_psum, a.blk_z, a.bias_select);
  return hipGetLastError();
}

template <typename Tin, int EP, int NW>
hipError_t launch_route_narrow(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  hipLaunchKernelGGL((route_narrow_kernel<Tin, EP, NW>), dim3(rt.NB), dim3(NW * 64), 0, st,
                     static_cast<const Tin*>(a.h), a.Wr, a.br, a.noise, a.T, a.d, a.E, a.K, a.gate, a.topk_idx,
                     a.topk_gate, a.logits, a.blk_hist, a.blk_psum, a.blk_z, a.bias_select);
  return hipGetLastError();
}

template <typename Tin, int EP>
hipError_t launch_route_narrow_nw(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  return launch_route_narrow<Tin, EP, kNarrowNW>(a, rt, st);
}

template <typename Tin>
hipError_t launch_route_dtype(const RouteArgs& a, const RouteTiling& rt, hipStream_t st) {
  if (rt.NW > 0) {  // narrow layout
    return rt.EP == 8 ? launch_route_narrow_nw<Tin, 8>(a, rt, st) : launch_route_narrow_nw<Tin, 16>(a, rt, st);
  }
  switch (rt.EP) {  // wide layout: wide_tb<EP>() tokens x EP experts per block of 256 threads
    case 8: return launch_route_wide<Tin, 8, WideCfg<8>::TE, WideCfg<8>::TPT, WideCfg<8>::BK, 2>(a, rt, st);
    case 16: return launch_route_wide<Tin, 16, WideCfg<16>::TE, WideCfg<16>::TPT, WideCfg<16>::BK, 2>(a, rt, st);
    case 32: return launch_route_mfma<Tin, 32>(a, rt, st);
    default: return launch_route_mfma<Tin, 64>(a, rt, st);
  }
}

}  // namespace

// Narrow layout for small batches of few experts (T <= 256, E <= 16), where the
// wide layout leaves most compute units idle: one token per wave, 4 waves per
// block. Otherwise the wide layout (up to 16 experts, wide_tb<EP>() tokens per
// block) or the MFMA layout (17..64 experts, kMfmaTB tokens per block).
constexpr int64_t kNarrowMaxT = 256;

RouteTiling route_tiling(int64_t T, int64_t E) {
  RouteTiling rt;
  rt.EP = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
  if (rt.EP <= 16 && T <= kNarrowMaxT) {
    rt.NW = kNarrowNW;
    rt.TB = kNarrowNW;
  } else {
    rt.NW = 0;  // wide or broadcast layout
    rt.TB = rt.EP == 8 ? wide_tb<8>() : rt.EP == 16 ? wide_tb<16>() : kMfmaTB;
  }
  rt.NB = static_cast<int>((T + rt.TB - 1) / rt.TB);
  return rt;
}

hipError_t launch_route(const RouteArgs& a, const RouteTiling& rt, bool bf16, hipStream_t st) {
  return bf16 ? launch_route_dtype<bf16_t>(a, rt, st) : launch_route_dtype<float>(a, rt, st);
}

hipError_t launch_hist(const int32_t* topk_idx, int T, int E, int K, const RouteTiling& rt,
                       int32_t* blk_hist, hipStream_t st) {
  hipLaunchKernelGGL(hist_kernel, dim3(rt.NB), dim3(256), 0, st, topk_idx, T, E, K, rt.TB, blk_hist);
  return hipGetLastError();
}

hipError_t launch_finalize(const int32_t* blk_hist, const float* blk_psum, const float* blk_z, int NB, int T,
                           int E, int K, int32_t* blk_base, int32_t* counts, int32_t* offsets, float* prob_mean,
                           float* aux, float* z_loss, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kFinThreads), 0, st, blk_hist, blk_psum, blk_z, NB, T, E,
                     K, blk_base, counts, offsets, prob_mean, aux, z_loss);
  return hipGetLastError();
}

hipError_t launch_zero_outputs(int E, int32_t* counts, int32_t* offsets, float* prob_mean, float* aux,
                               float* z_loss, hipStream_t st) {
  hipLaunchKernelGGL(zero_outputs_kernel, dim3(1), dim3(128), 0, st, E, counts, offsets, prob_mean, aux, z_loss);
  return hipGetLastError();
}

}  // namespace moe

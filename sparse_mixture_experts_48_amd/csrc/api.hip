// C-ABI of the MoE layer (declared in include/moe.h): argument validation,
// workspace carving and kernel launches on the caller's stream.
//
// Nothing here allocates device memory or synchronises the host (the trace
// functions aside). Every entry point validates all arguments before its first
// HIP call, so an invalid call leaves outputs and the stream untouched.
#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>
#include <vector>

#include "moe.h"
#include "kernels.h"

// Scratch of moe_forward_noalloc: one array per GPU, held from the library's
// first call on that GPU until the process ends. In host code `scratch` names
// a host-side stand-in, never the device memory: kernels and copies get the
// address hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
hipError_t launch_gemm1_bf16(const FfnArgs& f, hipStream_t st);
hipError_t launch_gemm2_bf16(const FfnArgs& f, hipStream_t st);
hipError_t launch_gemm1_f32(const FfnArgs& f, hipStream_t st);
hipError_t launch_gemm2_f32(const FfnArgs& f, hipStream_t st);

hipError_t launch_gemm1(const FfnArgs& f, hipStream_t st) {
  return f.bf16 ? launch_gemm1_bf16(f, st) : launch_gemm1_f32(f, st);
}
hipError_t launch_gemm2(const FfnArgs& f, hipStream_t st) {
  return f.bf16 ? launch_gemm2_bf16(f, st) : launch_gemm2_f32(f, st);
}
}  // namespace moe

namespace {

using moe::RouteTiling;

constexpr int64_t kMaxInt = 2147483647;
// Operand matrices (h, grouped rows, hidden activations, one expert's weight
// matrix) hold at most 2^31 - 2^22 elements and d, width are at most 2^20, so that
// 32-bit element offsets, and the byte offsets of the bfloat16 GEMMs' buffer
// loads (row offset + k offset), never wrap.
constexpr int64_t kMaxElems = (int64_t{1} << 31) - (int64_t{1} << 22);
constexpr int64_t kMaxDim = int64_t{1} << 20;

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Plan {
  RouteTiling rt;
  size_t blk_hist, blk_psum, blk_base, blk_z;
  size_t topk_idx, topk_gate, token_slot, slot_token;
  size_t counts, offsets, pmean, aux;
  size_t act, o_perm, tail_part;
  size_t total;
};

Plan make_plan(const moe_desc& d) {
  Plan p{};
  p.rt = moe::route_tiling(d.T, d.E);
  const size_t S = static_cast<size_t>(d.T) * d.K;
  const size_t bpe = d.dtype == MOE_BF16 ? 2 : 4;
  const size_t nbe = static_cast<size_t>(p.rt.NB) * d.E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p.blk_hist = take(nbe * 4);
  p.blk_psum = take(nbe * 4);
  p.blk_base = take(nbe * 4);
  p.blk_z = take(static_cast<size_t>(p.rt.NB) * 4);
  p.topk_idx = take(S * 4);
  p.topk_gate = take(S * 4);
  p.token_slot = take(S * 4);
  p.slot_token = take(S * 4);
  p.counts = take(d.E * 4);
  p.offsets = take((d.E + 1) * 4);
  p.pmean = take(d.E * 4);
  p.aux = take(4);
  p.act = take(S * d.width * bpe);
  p.o_perm = take(d.K > 1 || d.capacity > 0 ? S * d.d * 4 : 0);  // K = 1 dropless writes y directly
  // float32 partial rows of the second GEMM's split tails (moe_expert_ffn never
  // fuses the scatter, so the region is sized as if it did not)
  const int64_t max_rows = std::min<int64_t>(d.T, d.capacity > 0 ? d.capacity : INT_MAX);
  p.tail_part = take(d.dtype == MOE_BF16 ? moe::gemm2_tail_bytes(static_cast<int>(S), static_cast<int>(d.E),
                                                                   static_cast<int>(d.d), static_cast<int>(d.width),
                                                                   static_cast<int>(max_rows), false)
                                         : 0);
  p.total = off;
  return p;
}

// Workspace of moe_backward (bfloat16 layers). Zw = width of the first GEMM's
// pre-activations (2 width for SwiGLU); ldk = row length of the transposed
// per-slot operands: every expert's slots padded to a multiple of 64.
struct BwdPlan {
  RouteTiling rt;
  int64_t S, Zw, ldk;
  int nwr;
  size_t blk_hist, blk_psum, blk_base, blk_z, topk_idx, topk_gate, token_slot, slot_token, counts, offsets, aux,
      logits;
  size_t z, a, rgate, dyb, dgp, dgs, dO, dZ, dX, kofs, xT, dl, wr_part;
  size_t dx_tail;  // float32 partial rows of the dX GEMM's split tails (bfloat16 layers)
  size_t u;  // float32 layers: dy W2 of the grouped rows
  size_t total;
};

BwdPlan make_bwd_plan(const moe_desc& d) {
  BwdPlan p{};
  p.rt = moe::route_tiling(d.T, d.E);
  p.S = d.T * d.K;
  p.Zw = d.act == MOE_ACT_SWIGLU ? 2 * d.width : d.width;
  p.ldk = 64 * ((p.S + 63) / 64 + d.E);
  p.nwr = moe::dwr_chunks(static_cast<int>(d.T));
  const size_t S = static_cast<size_t>(p.S), nbe = static_cast<size_t>(p.rt.NB) * d.E;
  const size_t dd = static_cast<size_t>(d.d), w = static_cast<size_t>(d.width), Zw = static_cast<size_t>(p.Zw);
  const size_t E = static_cast<size_t>(d.E), ldk = static_cast<size_t>(p.ldk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p.blk_hist = take(nbe * 4);
  p.blk_psum = take(nbe * 4);
  p.blk_base = take(nbe * 4);
  p.blk_z = take(static_cast<size_t>(p.rt.NB) * 4);
  p.topk_idx = take(S * 4);
  p.topk_gate = take(S * 4);
  p.token_slot = take(S * 4);
  p.slot_token = take(S * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.aux = take(4);
  p.logits = take(static_cast<size_t>(d.T) * E * 4);
  if (d.dtype == MOE_F32) {  // float32 intermediates, no transposed copies
    p.z = take(S * Zw * 4);
    p.a = take(S * w * 4);
    p.rgate = take(S * 4);
    p.dyb = take(S * 4);
    p.dgs = take(S * 4);
    p.dO = take(S * dd * 4);
    p.u = take(S * w * 4);
    p.dZ = take(S * Zw * 4);
    p.dX = take(S * dd * 4);
    p.dl = take(static_cast<size_t>(d.T) * E * 4);
    p.wr_part = take(static_cast<size_t>(p.nwr) * dd * E * 4);
    p.total = off;
    return p;
  }
  p.z = take(S * Zw * 2);
  p.a = take(S * w * 2);
  p.rgate = take(S * 4);
  p.dyb = take(S * 4);
  p.dgp = take(static_cast<size_t>((w + moe::kDgpColsHost - 1) / moe::kDgpColsHost) * S * 4);
  p.dgs = take(S * 4);
  p.dO = take(S * dd * 2);
  p.dZ = take(S * Zw * 2);
  p.dX = take(S * dd * 4);
  p.kofs = take((E + 1) * 4);
  p.xT = take(dd * ldk * 2);
  p.dl = take(static_cast<size_t>(d.T) * E * 4);
  p.wr_part = take(static_cast<size_t>(p.nwr) * dd * E * 4);
  p.dx_tail = take(moe::bwd_dx_tail_bytes(static_cast<int>(S), static_cast<int>(E), static_cast<int>(dd),
                                          static_cast<int>(Zw)));
  p.total = off;
  return p;
}

// Shapes moe_backward supports beyond check_desc: every transposed or widened
// operand within the 32-bit offset range of the GEMMs.
int check_bwd_desc(const moe_desc& d) {
  const int64_t S = d.T * d.K, Zw = d.act == MOE_ACT_SWIGLU ? 2 * d.width : d.width;
  const int64_t ldk = 64 * ((S + 63) / 64 + d.E);
  if (S > 0 && S > kMaxElems / Zw) return MOE_ERR_UNSUPPORTED;
  if (ldk > kMaxElems / d.d) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Rows an expert processes at most: its capacity, or every row when dropless.
int cap_of(const moe_desc& d) { return d.capacity > 0 ? d.capacity : INT_MAX; }

int check_desc(const moe_desc* d) {
  if (d == nullptr) return MOE_ERR_NULL;
  if (d->T < 0 || d->d < 1 || d->width < 1 || d->E < 1 || d->K < 1 || d->K > d->E) return MOE_ERR_SHAPE;
  if (d->E > 64 || d->K > 8 || d->d % 8 != 0 || d->width % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->act != MOE_ACT_GELU && d->act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (d->gate != MOE_GATE_RENORM && d->gate != MOE_GATE_RAW) return MOE_ERR_UNSUPPORTED;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->capacity < 0) return MOE_ERR_SHAPE;
  if (d->bias_mode != MOE_BIAS_LOGITS && d->bias_mode != MOE_BIAS_SELECT) return MOE_ERR_UNSUPPORTED;
  if (d->T > kMaxInt / d->K || d->d > kMaxDim || d->width > kMaxDim) return MOE_ERR_UNSUPPORTED;
  const int64_t S = d->T * d->K;
  if (S > 0 && (S > kMaxElems / d->d || S > kMaxElems / d->width)) return MOE_ERR_UNSUPPORTED;
  if (d->d > kMaxElems / d->width) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A tensor pointer: NULL only when the tensor has no elements; 16-byte aligned.
int check_ptr(const void* p, bool has_elements) {
  if (p == nullptr) return has_elements ? MOE_ERR_NULL : MOE_OK;
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_ws(const Plan& pl, const void* ws, size_t ws_bytes) {
  if (ws_bytes < pl.total) return MOE_ERR_WORKSPACE;
  if (pl.total > 0 && ws == nullptr) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

#define MOE_CHECK(expr)              \
  do {                               \
    const int _s = (expr);           \
    if (_s != MOE_OK) return _s;     \
  } while (0)

int check_experts(const moe_desc& d, const void* W1, const void* b1, const void* W3, const void* W2,
                  const void* b2) {
  MOE_CHECK(check_ptr(W1, true));
  MOE_CHECK(check_ptr(W2, true));
  if (d.act == MOE_ACT_SWIGLU) {
    if (W3 == nullptr) return MOE_ERR_UNSUPPORTED;
    MOE_CHECK(check_ptr(W3, true));
  }
  MOE_CHECK(check_ptr(b1, false));
  MOE_CHECK(check_ptr(b2, false));
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------------------- tracing

struct TraceState {
  bool on = false;
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int32_t> kid;
};
TraceState g_trace;

template <typename F>
hipError_t traced(int kid, hipStream_t st, F&& launch) {
  if (!g_trace.on || g_trace.n >= g_trace.cap) return launch();
  const int i = g_trace.n++;
  g_trace.kid[i] = kid;
  (void)hipEventRecord(g_trace.ev[2 * i], st);
  const hipError_t err = launch();
  (void)hipEventRecord(g_trace.ev[2 * i + 1], st);
  return err;
}


#define MOE_LAUNCH(kid, st, call)                                 \
  do {                                                            \
    const hipError_t _e = traced((kid), (st), [&] { return call; }); \
    if (_e != hipSuccess) return MOE_ERR_HIP;                     \
  } while (0)

// Every argument of moe_forward / moe_forward_noalloc except the workspace.
int check_forward(const moe_desc* desc, const void* h, const float* W_r, const float* b_r, const void* W1,
                  const void* b1, const void* W3, const void* W2, const void* b2, const void* y,
                  const float* aux_loss, const int32_t* expert_counts, const float* noise, const float* z_loss) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  const bool any = d.T > 0;
  MOE_CHECK(check_ptr(h, any));
  MOE_CHECK(check_ptr(W_r, true));
  MOE_CHECK(check_ptr(b_r, false));
  MOE_CHECK(check_experts(d, W1, b1, W3, W2, b2));
  MOE_CHECK(check_ptr(y, any));
  MOE_CHECK(check_ptr(aux_loss, false));
  MOE_CHECK(check_ptr(expert_counts, false));
  MOE_CHECK(check_ptr(noise, false));
  MOE_CHECK(check_ptr(z_loss, false));
  return MOE_OK;
}

// The whole layer on stream st, with scratch at ws (laid out by pl); the
// arguments have passed check_forward.
int enqueue_forward(const moe_desc& d, const Plan& pl, const void* h, const float* W_r, const float* b_r,
                    const void* W1, const void* b1, const void* W3, const void* W2, const void* b2, void* y,
                    float* aux_loss, int32_t* expert_counts, const float* noise, float* z_loss, void* ws,
                    hipStream_t st) {
  const bool any = d.T > 0;
  if (!any) {
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_zero_outputs(d.E, expert_counts, nullptr, nullptr, aux_loss, z_loss, st));
    return MOE_OK;
  }
  const int T = static_cast<int>(d.T), E = static_cast<int>(d.E), K = static_cast<int>(d.K);
  const bool bf16 = d.dtype == MOE_BF16;
  int32_t* topk_idx = at<int32_t>(ws, pl.topk_idx);
  float* topk_gate = at<float>(ws, pl.topk_gate);
  int32_t* blk_hist = at<int32_t>(ws, pl.blk_hist);
  float* blk_psum = at<float>(ws, pl.blk_psum);
  int32_t* offsets = at<int32_t>(ws, pl.offsets);
  int32_t* slot_token = at<int32_t>(ws, pl.slot_token);
  int32_t* token_slot = at<int32_t>(ws, pl.token_slot);
  int32_t* counts = expert_counts != nullptr ? expert_counts : at<int32_t>(ws, pl.counts);

  moe::RouteArgs ra{h, W_r, b_r, T, static_cast<int>(d.d), E, K, d.gate, topk_idx, topk_gate, nullptr,
                    blk_hist, blk_psum};
  ra.bias_select = d.bias_mode == MOE_BIAS_SELECT && b_r != nullptr;
  ra.noise = noise;
  ra.blk_z = z_loss != nullptr ? at<float>(ws, pl.blk_z) : nullptr;
  MOE_LAUNCH(MOE_K_ROUTE, st, moe::launch_route(ra, pl.rt, bf16, st));
  const size_t row_bytes = static_cast<size_t>(d.d) * (bf16 ? 2 : 4);
  const int cap = cap_of(d);
  {  // statistics and grouping in one launch
    moe::FinArgs fin;
    fin.blk_hist = blk_hist;
    fin.blk_psum = blk_psum;
    fin.blk_z = ra.blk_z;
    fin.NB = pl.rt.NB;
    fin.counts = counts;
    fin.offsets = offsets;
    fin.aux = aux_loss;
    fin.z_loss = z_loss;
    MOE_LAUNCH(MOE_K_PERMUTE, st,
               moe::launch_finalize_permute(fin, topk_idx, T, E, K, cap, pl.rt, h, row_bytes, nullptr, slot_token,
                                            token_slot, st));
  }
  // GEMM1 reads the rows of h through slot_token: the grouped copy of h is never written.
  moe::FfnArgs f{};
  f.S = T * K;
  f.d = static_cast<int>(d.d);
  f.E = E;
  f.K = K;
  f.width = static_cast<int>(d.width);
  f.act = d.act;
  f.bf16 = bf16;
  f.x = h;
  f.x_rows = slot_token;
  f.offsets = offsets;
  f.W1 = W1; f.b1 = b1; f.W3 = W3; f.W2 = W2; f.b2 = b2;
  f.a = at<char>(ws, pl.act);
  f.o_perm = at<float>(ws, pl.o_perm);
  f.tail_part = at<float>(ws, pl.tail_part);
  f.fused_y = K == 1 && d.capacity == 0;  // with drops, the combine writes the tokens that lost their slot
  f.y = y;
  f.slot_token = slot_token;
  f.topk_gate = topk_gate;
  f.cap = cap;
  f.max_rows_per_expert = std::min(T, cap);
  MOE_LAUNCH(MOE_K_GEMM1, st, moe::launch_gemm1(f, st));
  MOE_LAUNCH(MOE_K_GEMM2, st, moe::launch_gemm2(f, st));
  if (!f.fused_y) {
    MOE_LAUNCH(MOE_K_COMBINE, st, moe::launch_combine(f.o_perm, token_slot, topk_gate, T, f.d, K, bf16, y, st));
  }
  return MOE_OK;
}

// Backward pass of a float32 layer after the routing and grouping (shared
// with the bfloat16 path): the same gradients from float32 kernels, with no
// transposed copies (the GEMMs read the weights with k as the row index).
int backward_f32(const moe_desc& d, const BwdPlan& pl, const void* h, const float* W_r, const float* b_r,
                 const void* W1, const void* b1, const void* W3, const void* W2, const void* b2, const void* dy,
                 float daux, float dz, void* dh, float* dW_r, float* db_r, float* dW1, float* db1, float* dW3,
                 float* dW2, float* db2, void* ws, hipStream_t st) {
  const int T = static_cast<int>(d.T), E_ = static_cast<int>(d.E), K = static_cast<int>(d.K);
  const int D = static_cast<int>(d.d), Wd = static_cast<int>(d.width), S = static_cast<int>(pl.S);
  const int Zw = static_cast<int>(pl.Zw);
  const bool swiglu = d.act == MOE_ACT_SWIGLU;
  const int cap = cap_of(d);
  const int bias_select = d.bias_mode == MOE_BIAS_SELECT && b_r != nullptr;
  const int32_t* topk_idx = at<int32_t>(ws, pl.topk_idx);
  const float* topk_gate = at<float>(ws, pl.topk_gate);
  const int32_t* offsets = at<int32_t>(ws, pl.offsets);
  const int32_t* slot_token = at<int32_t>(ws, pl.slot_token);
  const int32_t* token_slot = at<int32_t>(ws, pl.token_slot);
  const int32_t* counts = at<int32_t>(ws, pl.counts);
  const float* logits = at<float>(ws, pl.logits);
  float* z = at<float>(ws, pl.z);
  float* a = at<float>(ws, pl.a);
  float* rgate = at<float>(ws, pl.rgate);
  float* dyb = at<float>(ws, pl.dyb);
  float* dgs = at<float>(ws, pl.dgs);
  float* dO = at<float>(ws, pl.dO);
  float* u = at<float>(ws, pl.u);
  float* dZ = at<float>(ws, pl.dZ);
  float* dX = at<float>(ws, pl.dX);
  float* dl = at<float>(ws, pl.dl);

  moe::FfnArgs f{};
  f.S = S;
  f.d = D;
  f.E = E_;
  f.K = K;
  f.width = Wd;
  f.act = d.act;
  f.bf16 = false;
  f.x = h;
  f.x_rows = slot_token;
  f.offsets = offsets;
  f.W1 = W1; f.b1 = b1; f.W3 = W3; f.W2 = W2; f.b2 = b2;
  f.cap = cap;
  MOE_LAUNCH(MOE_K_GEMM1, st, moe::launch_bwd_z_f32(f, z, a, st));
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_dout(dy, token_slot, topk_idx, topk_gate, b2, T, D, K, dO, rgate, dyb, false, st));
  // u = dy W2 for every grouped row (W2 [E][d][width]: k = d is its row index)
  MOE_LAUNCH(MOE_K_GEMM2, st,
             moe::launch_bwd_grouped_f32(static_cast<const float*>(dy), slot_token, D, S, offsets, cap, E_,
                                         static_cast<const float*>(W2), nullptr, 0, Wd, D, u, st));
  MOE_LAUNCH(MOE_K_BWD, st, moe::launch_dz_f32(u, z, a, rgate, S, Wd, swiglu ? 1 : 0, dZ, dgs, st));
  // dX = dZ [W1; W3] (W1, W3 [E][width][d]: k = width is their row index)
  MOE_LAUNCH(MOE_K_GEMM1, st,
             moe::launch_bwd_grouped_f32(dZ, nullptr, Zw, S, offsets, cap, E_, static_cast<const float*>(W1),
                                         swiglu ? static_cast<const float*>(W3) : nullptr, Wd, D, Wd, dX, st));
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_router_backward(logits, b_r, bias_select, topk_idx, topk_gate, dgs, dyb, token_slot,
                                         counts, T, E_, K, d.gate, daux, dz, dl, st));
  MOE_LAUNCH(MOE_K_BWD, st, moe::launch_dh(dX, token_slot, dl, W_r, T, D, E_, K, dh, false, st));
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_dwr(h, dl, T, D, E_, at<float>(ws, pl.wr_part), dW_r, bias_select ? nullptr : db_r, false,
                             st));
  if (bias_select) MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(db_r, static_cast<size_t>(E_) * 4, st));
  // weight gradients: dW2[e] = sum_s dO[s]^T a[s]; [dW1; dW3][e] = sum_s dZ[s]^T x[s]
  MOE_LAUNCH(MOE_K_WGRAD, st,
             moe::launch_bwd_wgrad_f32(dO, D, a, nullptr, Wd, offsets, S, cap, E_, dW2, nullptr, D, st));
  MOE_LAUNCH(MOE_K_WGRAD, st,
             moe::launch_bwd_wgrad_f32(dZ, Zw, static_cast<const float*>(h), slot_token, D, offsets, S, cap, E_, dW1,
                                       dW3, Wd, st));
  if (db1 != nullptr)
    MOE_LAUNCH(MOE_K_BWD, st, moe::launch_group_colsum(dZ, Wd, offsets, E_, S, cap, db1, false, st));
  if (db2 != nullptr)
    MOE_LAUNCH(MOE_K_BWD, st, moe::launch_group_colsum(dO, D, offsets, E_, S, cap, db2, false, st));
  return MOE_OK;
}

// ---------------------------------------------------------------------------- static scratch

constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id; null until looked up

// Device address of the current GPU's scratch array (looked up once per device).
int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (static_cast<size_t>(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(static_cast<size_t>(dev) + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MOE_ERR_HIP;
    if (reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: invalid layer shape";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape, type or alignment not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small or misaligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown moe_status";
  }
}

const char* moe_kernel_name(int kernel_id) {
  switch (kernel_id) {
    case MOE_K_ROUTE: return "route";
    case MOE_K_FINALIZE: return "finalize";
    case MOE_K_HIST: return "hist";
    case MOE_K_PERMUTE: return "permute";
    case MOE_K_GEMM1: return "gemm1";
    case MOE_K_GEMM2: return "gemm2";
    case MOE_K_COMBINE: return "combine";
    case MOE_K_ZERO: return "zero";
    case MOE_K_BWD: return "backward";
    case MOE_K_WGRAD: return "wgrad";
    default: return "unknown";
  }
}

int moe_capacity_slots(double factor, int64_t T, int64_t K, int64_t E, int32_t* slots) {
  if (slots == nullptr) return MOE_ERR_NULL;
  if (!std::isfinite(factor) || factor < 0.0 || T < 0 || K < 1 || E < 1) return MOE_ERR_SHAPE;
  const double x = factor * static_cast<double>(T) * static_cast<double>(K) / static_cast<double>(E);
  const double r = std::nearbyint(x);
  const double c = (std::fabs(x - r) <= 1e-9 * std::max(1.0, std::fabs(x))) ? r : std::ceil(x);
  if (c > static_cast<double>(kMaxInt)) return MOE_ERR_UNSUPPORTED;
  *slots = static_cast<int32_t>(c);
  return MOE_OK;
}

int moe_workspace_size(const moe_desc* desc, size_t* bytes) {
  MOE_CHECK(check_desc(desc));
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = make_plan(*desc).total;
  return MOE_OK;
}

int moe_route(const moe_desc* desc, const void* h, const float* W_r, const float* b_r, int32_t* topk_idx,
              float* topk_gate, int32_t* expert_counts, float* prob_mean, float* aux_loss, float* logits,
              const float* noise, float* z_loss, void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  const bool any = d.T > 0;
  MOE_CHECK(check_ptr(h, any));
  MOE_CHECK(check_ptr(W_r, true));
  MOE_CHECK(check_ptr(b_r, false));
  MOE_CHECK(check_ptr(topk_idx, any));
  MOE_CHECK(check_ptr(topk_gate, any));
  MOE_CHECK(check_ptr(expert_counts, true));
  MOE_CHECK(check_ptr(prob_mean, false));
  MOE_CHECK(check_ptr(aux_loss, false));
  MOE_CHECK(check_ptr(logits, false));
  MOE_CHECK(check_ptr(noise, false));
  MOE_CHECK(check_ptr(z_loss, false));
  const Plan pl = make_plan(d);
  MOE_CHECK(check_ws(pl, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!any) {
    MOE_LAUNCH(MOE_K_ZERO, st,
               moe::launch_zero_outputs(d.E, expert_counts, nullptr, prob_mean, aux_loss, z_loss, st));
    return MOE_OK;
  }
  moe::RouteArgs ra{h, W_r, b_r, static_cast<int>(d.T), static_cast<int>(d.d), static_cast<int>(d.E),
                    static_cast<int>(d.K), d.gate, topk_idx, topk_gate, logits,
                    at<int32_t>(ws, pl.blk_hist), at<float>(ws, pl.blk_psum)};
  ra.bias_select = d.bias_mode == MOE_BIAS_SELECT && b_r != nullptr;
  ra.noise = noise;
  ra.blk_z = z_loss != nullptr ? at<float>(ws, pl.blk_z) : nullptr;
  MOE_LAUNCH(MOE_K_ROUTE, st, moe::launch_route(ra, pl.rt, d.dtype == MOE_BF16, st));
  MOE_LAUNCH(MOE_K_FINALIZE, st,
             moe::launch_finalize(ra.blk_hist, ra.blk_psum, ra.blk_z, pl.rt.NB, ra.T, ra.E, ra.K, nullptr,
                                  expert_counts, nullptr, prob_mean, aux_loss, z_loss, st));
  return MOE_OK;
}

int moe_permute(const moe_desc* desc, const int32_t* topk_idx, const void* h, int32_t* expert_offsets,
                int32_t* slot_token, int32_t* token_slot, void* h_perm, void* ws, size_t ws_bytes,
                void* stream) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  const bool any = d.T > 0;
  MOE_CHECK(check_ptr(topk_idx, any));
  MOE_CHECK(check_ptr(h, any));
  MOE_CHECK(check_ptr(expert_offsets, true));
  MOE_CHECK(check_ptr(slot_token, any));
  MOE_CHECK(check_ptr(token_slot, any));
  MOE_CHECK(check_ptr(h_perm, any));
  const Plan pl = make_plan(d);
  MOE_CHECK(check_ws(pl, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!any) {
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_zero_outputs(d.E, nullptr, expert_offsets, nullptr, nullptr, nullptr, st));
    return MOE_OK;
  }
  const int T = static_cast<int>(d.T), E = static_cast<int>(d.E), K = static_cast<int>(d.K);
  int32_t* blk_hist = at<int32_t>(ws, pl.blk_hist);
  int32_t* blk_base = at<int32_t>(ws, pl.blk_base);
  const size_t row_bytes = static_cast<size_t>(d.d) * (d.dtype == MOE_BF16 ? 2 : 4);
  MOE_LAUNCH(MOE_K_HIST, st, moe::launch_hist(topk_idx, T, E, K, pl.rt, blk_hist, st));
  MOE_LAUNCH(MOE_K_FINALIZE, st,
             moe::launch_finalize(blk_hist, nullptr, nullptr, pl.rt.NB, T, E, K, blk_base, nullptr, expert_offsets,
                                  nullptr, nullptr, nullptr, st));
  MOE_LAUNCH(MOE_K_PERMUTE, st,
             moe::launch_permute(topk_idx, blk_base, expert_offsets, T, E, K, cap_of(d), pl.rt, h, row_bytes,
                                 h_perm, slot_token, token_slot, st));
  return MOE_OK;
}

int moe_expert_ffn(const moe_desc* desc, const void* h_perm, const int32_t* expert_offsets, const void* W1,
                   const void* b1, const void* W3, const void* W2, const void* b2, float* o_perm, void* ws,
                   size_t ws_bytes, void* stream) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  const bool any = d.T > 0;
  MOE_CHECK(check_ptr(h_perm, any));
  MOE_CHECK(check_ptr(expert_offsets, true));
  MOE_CHECK(check_experts(d, W1, b1, W3, W2, b2));
  MOE_CHECK(check_ptr(o_perm, any));
  const Plan pl = make_plan(d);
  MOE_CHECK(check_ws(pl, ws, ws_bytes));
  if (!any) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::FfnArgs f{};
  f.S = static_cast<int>(d.T * d.K);
  f.d = static_cast<int>(d.d);
  f.E = static_cast<int>(d.E);
  f.K = static_cast<int>(d.K);
  f.width = static_cast<int>(d.width);
  f.act = d.act;
  f.bf16 = d.dtype == MOE_BF16;
  f.x = h_perm;
  f.offsets = expert_offsets;
  f.W1 = W1; f.b1 = b1; f.W3 = W3; f.W2 = W2; f.b2 = b2;
  f.a = at<char>(ws, pl.act);
  f.o_perm = o_perm;
  f.tail_part = at<float>(ws, pl.tail_part);
  f.fused_y = false;
  f.cap = cap_of(d);
  f.max_rows_per_expert = static_cast<int>(std::min<int64_t>(d.T, f.cap));
  MOE_LAUNCH(MOE_K_GEMM1, st, moe::launch_gemm1(f, st));
  MOE_LAUNCH(MOE_K_GEMM2, st, moe::launch_gemm2(f, st));
  return MOE_OK;
}

int moe_combine(const moe_desc* desc, const float* o_perm, const int32_t* token_slot, const float* topk_gate,
                void* y, void* stream) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  const bool any = d.T > 0;
  MOE_CHECK(check_ptr(o_perm, any));
  MOE_CHECK(check_ptr(token_slot, any));
  MOE_CHECK(check_ptr(topk_gate, any));
  MOE_CHECK(check_ptr(y, any));
  if (!any) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_LAUNCH(MOE_K_COMBINE, st,
             moe::launch_combine(o_perm, token_slot, topk_gate, static_cast<int>(d.T), static_cast<int>(d.d),
                                 static_cast<int>(d.K), d.dtype == MOE_BF16, y, st));
  return MOE_OK;
}

int moe_forward(const moe_desc* desc, const void* h, const float* W_r, const float* b_r, const void* W1,
                const void* b1, const void* W3, const void* W2, const void* b2, void* y, float* aux_loss,
                int32_t* expert_counts, const float* noise, float* z_loss, void* ws, size_t ws_bytes,
                void* stream) {
  MOE_CHECK(check_forward(desc, h, W_r, b_r, W1, b1, W3, W2, b2, y, aux_loss, expert_counts, noise, z_loss));
  const Plan pl = make_plan(*desc);
  MOE_CHECK(check_ws(pl, ws, ws_bytes));
  return enqueue_forward(*desc, pl, h, W_r, b_r, W1, b1, W3, W2, b2, y, aux_loss, expert_counts, noise, z_loss, ws,
                         static_cast<hipStream_t>(stream));
}

int moe_forward_noalloc(const moe_desc* desc, const void* h, const float* W_r, const float* b_r, const void* W1,
                        const void* b1, const void* W3, const void* W2, const void* b2, void* y, float* aux_loss,
                        int32_t* expert_counts, const float* noise, float* z_loss, void* stream) {
  MOE_CHECK(check_forward(desc, h, W_r, b_r, W1, b1, W3, W2, b2, y, aux_loss, expert_counts, noise, z_loss));
  const Plan pl = make_plan(*desc);
  if (pl.total > kNoallocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  MOE_CHECK(noalloc_scratch(&ws));
  return enqueue_forward(*desc, pl, h, W_r, b_r, W1, b1, W3, W2, b2, y, aux_loss, expert_counts, noise, z_loss, ws,
                         static_cast<hipStream_t>(stream));
}

int moe_backward_workspace_size(const moe_desc* desc, size_t* bytes) {
  MOE_CHECK(check_desc(desc));
  MOE_CHECK(check_bwd_desc(*desc));
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = make_bwd_plan(*desc).total;
  return MOE_OK;
}

int moe_backward(const moe_desc* desc, const void* h, const float* W_r, const float* b_r, const void* W1,
                 const void* b1, const void* W3, const void* W2, const void* b2, const void* dy, float daux,
                 const float* noise, float dz, void* dh, float* dW_r, float* db_r, float* dW1, float* db1,
                 float* dW3, float* dW2, float* db2, void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_CHECK(check_bwd_desc(d));
  const bool any = d.T > 0;
  const bool swiglu = d.act == MOE_ACT_SWIGLU;
  MOE_CHECK(check_ptr(h, any));
  MOE_CHECK(check_ptr(W_r, true));
  MOE_CHECK(check_ptr(b_r, false));
  MOE_CHECK(check_experts(d, W1, b1, W3, W2, b2));
  MOE_CHECK(check_ptr(dy, any));
  MOE_CHECK(check_ptr(dh, any));
  MOE_CHECK(check_ptr(dW_r, true));
  MOE_CHECK(check_ptr(db_r, false));
  MOE_CHECK(check_ptr(dW1, true));
  MOE_CHECK(check_ptr(dW2, true));
  MOE_CHECK(check_ptr(db1, false));
  MOE_CHECK(check_ptr(db2, false));
  if (swiglu) MOE_CHECK(check_ptr(dW3, true));
  if (swiglu && (db1 != nullptr || db2 != nullptr || b1 != nullptr || b2 != nullptr)) return MOE_ERR_UNSUPPORTED;
  if (!std::isfinite(daux) || !std::isfinite(dz)) return MOE_ERR_SHAPE;
  MOE_CHECK(check_ptr(noise, false));
  const BwdPlan pl = make_bwd_plan(d);
  if (ws_bytes < pl.total || ws == nullptr || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t E = static_cast<size_t>(d.E), dd = static_cast<size_t>(d.d), w = static_cast<size_t>(d.width);
  if (!any) {  // no tokens: every gradient is zero
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(dW_r, dd * E * 4, st));
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(db_r, E * 4, st));
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(dW1, E * w * dd * 4, st));
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(dW2, E * w * dd * 4, st));
    if (swiglu) MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(dW3, E * w * dd * 4, st));
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(db1, E * w * 4, st));
    MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(db2, E * dd * 4, st));
    return MOE_OK;
  }
  const int T = static_cast<int>(d.T), E_ = static_cast<int>(d.E), K = static_cast<int>(d.K);
  const int D = static_cast<int>(d.d), Wd = static_cast<int>(d.width), S = static_cast<int>(pl.S);
  const int Zw = static_cast<int>(pl.Zw), ldk = static_cast<int>(pl.ldk);
  const int cap = cap_of(d);
  const int act = swiglu ? 1 : 0;
  int32_t* topk_idx = at<int32_t>(ws, pl.topk_idx);
  float* topk_gate = at<float>(ws, pl.topk_gate);
  int32_t* blk_hist = at<int32_t>(ws, pl.blk_hist);
  float* blk_psum = at<float>(ws, pl.blk_psum);
  int32_t* offsets = at<int32_t>(ws, pl.offsets);
  int32_t* slot_token = at<int32_t>(ws, pl.slot_token);
  int32_t* token_slot = at<int32_t>(ws, pl.token_slot);
  int32_t* counts = at<int32_t>(ws, pl.counts);
  float* logits = at<float>(ws, pl.logits);
  const int bias_select = d.bias_mode == MOE_BIAS_SELECT && b_r != nullptr;

  // forward: routing (with the logits), grouping, the expert GEMMs
  moe::RouteArgs ra{h, W_r, b_r, T, D, E_, K, d.gate, topk_idx, topk_gate, logits, blk_hist, blk_psum};
  ra.bias_select = bias_select;
  ra.noise = noise;
  const bool bf16 = d.dtype == MOE_BF16;
  MOE_LAUNCH(MOE_K_ROUTE, st, moe::launch_route(ra, pl.rt, bf16, st));
  moe::FinArgs fin;
  fin.blk_hist = blk_hist;
  fin.blk_psum = blk_psum;
  fin.NB = pl.rt.NB;
  fin.counts = counts;
  fin.offsets = offsets;
  fin.aux = at<float>(ws, pl.aux);
  MOE_LAUNCH(MOE_K_PERMUTE, st,
             moe::launch_finalize_permute(fin, topk_idx, T, E_, K, cap, pl.rt, h, dd * (bf16 ? 2 : 4), nullptr,
                                          slot_token, token_slot, st));
  if (d.dtype == MOE_F32)
    return backward_f32(d, pl, h, W_r, b_r, W1, b1, W3, W2, b2, dy, daux, dz, dh, dW_r, db_r, dW1, db1, dW3, dW2, db2,
                        ws, st);
  int32_t* kofs = at<int32_t>(ws, pl.kofs);
  MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_pad_offsets(offsets, E_, S, cap, kofs, st));
  moe::FfnArgs f{};
  f.S = S;
  f.d = D;
  f.E = E_;
  f.K = K;
  f.width = Wd;
  f.act = d.act;
  f.bf16 = true;
  f.x = h;
  f.x_rows = slot_token;
  f.offsets = offsets;
  f.W1 = W1; f.b1 = b1; f.W3 = W3; f.W2 = W2; f.b2 = b2;
  f.cap = cap;
  f.max_rows_per_expert = std::min(T, cap);
  void* z = at<char>(ws, pl.z);
  void* a = at<char>(ws, pl.a);
  MOE_LAUNCH(MOE_K_GEMM1, st, moe::launch_bwd_z_bf16(f, z, a, st));

  // backward through the combine, the second GEMM, the activation, the first
  // GEMM. The gate gradient dy . o = dy . (a W2^T + b2) is taken as
  // a . (dy W2) inside the dZ GEMM (which reduces dy W2 anyway) plus dy . b2,
  // so the expert outputs o are never recomputed.
  float* rgate = at<float>(ws, pl.rgate);
  float* dyb = at<float>(ws, pl.dyb);
  float* dgp = at<float>(ws, pl.dgp);
  float* dgs = at<float>(ws, pl.dgs);
  void* dO = at<char>(ws, pl.dO);
  void* dZ = at<char>(ws, pl.dZ);
  float* dX = at<float>(ws, pl.dX);
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_dout(dy, token_slot, topk_idx, topk_gate, b2, T, D, K, dO, rgate, dyb, true, st));
  // the dZ and dX GEMMs read W2 and [W1; W3] as stored, with k as the row index
  MOE_LAUNCH(MOE_K_GEMM2, st,
             moe::launch_bwd_dz_bf16(dy, T, slot_token, S, offsets, cap, E_, W2, Wd, D, z, act, rgate, a, dgp, dZ,
                                     st));
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_dgate_sum(dgp, (Wd + moe::kDgpColsHost - 1) / moe::kDgpColsHost, S, dgs, st));
  MOE_LAUNCH(MOE_K_GEMM1, st,
             moe::launch_bwd_dx_bf16(dZ, S, offsets, cap, E_, W1, swiglu ? W3 : nullptr, D, Wd, dX,
                                     at<float>(ws, pl.dx_tail), st));

  // router, dh, dW_r, db_r
  float* dl = at<float>(ws, pl.dl);
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_router_backward(logits, b_r, bias_select, topk_idx, topk_gate, dgs, dyb, token_slot,
                                         counts, T, E_, K, d.gate, daux, dz, dl, st));
  MOE_LAUNCH(MOE_K_BWD, st, moe::launch_dh(dX, token_slot, dl, W_r, T, D, E_, K, dh, true, st));
  MOE_LAUNCH(MOE_K_BWD, st,
             moe::launch_dwr(h, dl, T, D, E_, at<float>(ws, pl.wr_part), dW_r, bias_select ? nullptr : db_r, true,
                             st));
  if (bias_select) MOE_LAUNCH(MOE_K_ZERO, st, moe::launch_fill_zero(db_r, E * 4, st));

  // weight gradients: sums over each expert's kept grouped slots. dO, a and dZ
  // are read as written, with the slots as rows; h, gathered through
  // slot_token, is first transposed into [feature][slot] with every expert's
  // slots padded to whole 64-k stages.
  void* xT = at<char>(ws, pl.xT);
  MOE_LAUNCH(MOE_K_BWD, st, moe::launch_transpose_groups(h, slot_token, D, offsets, kofs, E_, S, cap, xT, ldk, st));
  MOE_LAUNCH(MOE_K_WGRAD, st,
             moe::launch_bwd_wgrad_bf16(dO, D, a, true, Wd, ldk, kofs, offsets, S, cap, E_, dW2, nullptr, D, st));
  MOE_LAUNCH(MOE_K_WGRAD, st,
             moe::launch_bwd_wgrad_bf16(dZ, Zw, xT, false, D, ldk, kofs, offsets, S, cap, E_, dW1, dW3, Wd, st));
  if (db1 != nullptr)
    MOE_LAUNCH(MOE_K_BWD, st, moe::launch_group_colsum(dZ, Wd, offsets, E_, S, cap, db1, true, st));
  if (db2 != nullptr)
    MOE_LAUNCH(MOE_K_BWD, st, moe::launch_group_colsum(dO, D, offsets, E_, S, cap, db2, true, st));
  return MOE_OK;
}

int moe_trace_enable(int capacity) {
  if (capacity < 1) return MOE_ERR_SHAPE;
  moe_trace_disable();
  g_trace.ev.assign(2 * static_cast<size_t>(capacity), nullptr);
  g_trace.kid.assign(capacity, -1);
  for (auto& e : g_trace.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      moe_trace_disable();
      return MOE_ERR_HIP;
    }
  }
  g_trace.cap = capacity;
  g_trace.n = 0;
  g_trace.on = true;
  return MOE_OK;
}

int moe_trace_read(int32_t* kernel_id, float* ms, int max, int* n) {
  if (kernel_id == nullptr || ms == nullptr || n == nullptr) return MOE_ERR_NULL;
  const int cnt = g_trace.n < max ? g_trace.n : max;
  if (g_trace.n > 0 && hipEventSynchronize(g_trace.ev[2 * (g_trace.n - 1) + 1]) != hipSuccess) return MOE_ERR_HIP;
  for (int i = 0; i < cnt; ++i) {
    kernel_id[i] = g_trace.kid[i];
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess) return MOE_ERR_HIP;
    ms[i] = t;
  }
  *n = cnt;
  g_trace.n = 0;
  return MOE_OK;
}

int moe_trace_disable(void) {
  for (auto& e : g_trace.ev)
    if (e != nullptr) (void)hipEventDestroy(e);
  g_trace.ev.clear();
  g_trace.kid.clear();
  g_trace.cap = 0;
  g_trace.n = 0;
  g_trace.on = false;
  return MOE_OK;
}

}  // extern "C"
